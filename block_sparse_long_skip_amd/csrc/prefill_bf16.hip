// bf16 skip-softmax prefill, d_qk = d_v = 128, 128-row query tiles, 64-key
// tiles, on gfx950 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Method: BLASST post (seeallochnaya, "BLASST: Dynamic BLocked Attention
// Sparsity via Softmax Thresholding"): key tiles in increasing order (paragraph
// "В чём идея"), online max with rescale (paragraph on FlashAttention 1), a
// tile dropped whole when its max is far below the running max and its V never
// read (paragraph beginning "BLASST предлагает"), tile 0 always processed
// (first figure). The drop test is one scalar threshold on the running-max
// statistics (digg thread "BLASST wins Best Paper at MLSys 2026").
//
// Layout. One workgroup of 4 waves per (batch, query head, query tile); wave w
// owns query rows [32w, 32w+32). Scores are computed transposed,
// S^T = K Q^T, so the MFMA result puts one query row in each lane column:
// lane l holds row 32w + (l & 31) and 32 of the tile's 64 keys (lane l ^ 32
// holds the other 32). Row max and row sum stay in-lane plus one lane swap.
// The output is accumulated transposed too, O^T = V^T P^T, so the rescale by
// exp(m_old - m_new) is a per-lane scalar. P^T feeds the second MFMA straight
// from the first MFMA's accumulators (the key order inside one MFMA's
// contraction is permuted to match the accumulator layout; the same
// permutation is applied to V^T, so the sum is unchanged).
//
// LDS: K tile row-major [64][128+8] bf16; V tile transposed [128][64+4] bf16
// (written transposed from coalesced global loads). The skip vote is a wave
// ballot over "this row keeps" plus an OR of the four waves' ballots through
// LDS, so every wave takes the same branch and V is loaded only after it.
#include "common.hpp"

namespace blasst {

namespace {
constexpr int D = 128;
constexpr int BR = 128;
constexpr int BC = 64;
constexpr int NT = 256;
constexpr int KP = D + 8;    // K tile pitch (bf16): 272 B rows, conflict-free b128 reads
constexpr int VP = BC + 4;   // V^T tile pitch (bf16): 136 B rows
}  // namespace

__global__ void __launch_bounds__(NT, 2) prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BC * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];
  __shared__ int votes[4];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // block -> (query tile, head): heaviest query tiles first; when the head
  // count is a multiple of 8, heads of one KV group land on the same XCD
  // (blocks are dealt to the 8 XCDs round-robin)
  const int nbh = a.B * a.Hq;
  const int i = a.nqt - 1 - (int)(blockIdx.x / nbh);
  int bh = (int)(blockIdx.x % nbh);
  if ((nbh & 7) == 0) bh = (bh & 7) * (nbh >> 3) + (bh >> 3);
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int kvh = hq / (a.Hq / a.Hkv);

  const uint16_t* qp = (const uint16_t*)a.q + b * a.qs0 + hq * a.qs1;
  const uint16_t* kp = (const uint16_t*)a.k + b * a.ks0 + kvh * a.ks1;
  const uint16_t* vp = (const uint16_t*)a.v + b * a.vs0 + kvh * a.vs1;

  const int row = i * BR + 32 * w + l32;  // this lane's query row
  const bool valid = row < a.Nq;
  const int qpos = row + (a.Nk - a.Nq);
  const int last_row = min(i * BR + BR - 1, a.Nq - 1);
  const int first_pos = i * BR + (a.Nk - a.Nq);  // key position of the tile's first row
  const int J = a.causal ? min(a.nkt, (last_row + a.Nk - a.Nq) / BC + 1) : a.nkt;

  // Q^T as the B operand: lane supplies Q[row][16kk + 8h .. +7]
  bf16x8_t qb[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (valid) v = load16(qp + (int64_t)row * a.qs2 + 16 * kk + 8 * h);
    qb[kk] = as_bf16x8(v);
  }

  f32x16_t o[4];  // O^T[dv = 32db + 8(r/4) + 4h + r%4][row]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = kNegInf, l = 0.f;
  int kept = 0;
  uint8_t* mrow = a.mask ? a.mask + ((int64_t)bh * a.nqt + i) * a.nkt : nullptr;

  for (int j = 0; j < J; ++j) {
    const int c0 = j * BC;
    __syncthreads();  // every wave is done with the previous K and V tiles
    // K tile -> LDS: 64 rows x 16 chunks of 16 B; thread: chunk t&15 of rows t/16 + 16r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kr = (t >> 4) + 16 * r, kc = (t & 15) * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (c0 + kr < a.Nk) v = load16(kp + (int64_t)(c0 + kr) * a.ks2 + kc);
      store16(&Ks[kr * KP + kc], v);
    }
    __syncthreads();

    // S^T = K Q^T: s[kb][r] is key c0 + 32kb + 8(r/4) + 4h + r%4 for this lane's row
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        bf16x8_t ka = as_bf16x8(*(const u32x4_t*)&Ks[(32 * kb + l32) * KP + 16 * kk + 8 * h]);
        s[kb] = mfma32x32x16(ka, qb[kk], s[kb]);
      }
    }
    // mask keys past Nk and (causal) keys after this row's position
    const bool need_mask = (c0 + BC > a.Nk) || (a.causal && c0 + BC - 1 > first_pos);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int col = c0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (col >= a.Nk || (a.causal && col > qpos)) s[kb][r] = kNegInf;
        }
    }
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = max_with_lane_xor32(mt);

    // vote: the tile is dropped only when every valid row is below the threshold
    float gap;
    if (mt == kNegInf) gap = kNegInf;
    else if (m == kNegInf) gap = __builtin_inff();
    else gap = mt - m;
    const bool lane_keep = valid && !(gap < a.thr_raw);
    const bool wave_keep = __any(lane_keep);
    if (lane == 0) votes[w] = wave_keep ? 1 : 0;
    __syncthreads();
    const bool keep = (j == 0) || (votes[0] | votes[1] | votes[2] | votes[3]);

    if (keep) {
      // V tile, only now: thread loads rows 4g..4g+3 (g = t/16) of dv chunk t&15
      // and writes them transposed, 4 keys (8 B) per dv row
      {
        const int g = t >> 4, cd = (t & 15) * 8;
        u32x4_t vr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = c0 + 4 * g + r;
          vr[r] = (u32x4_t){0u, 0u, 0u, 0u};
          if (key < a.Nk) vr[r] = load16(vp + (int64_t)key * a.vs2 + cd);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          u32x2_t lo = {pack_lo16(vr[0][p], vr[1][p]), pack_lo16(vr[2][p], vr[3][p])};
          u32x2_t hi = {pack_hi16(vr[0][p], vr[1][p]), pack_hi16(vr[2][p], vr[3][p])};
          *(u32x2_t*)&Vt[(cd + 2 * p) * VP + 4 * g] = lo;
          *(u32x2_t*)&Vt[(cd + 2 * p + 1) * VP + 4 * g] = hi;
        }
      }
      const float m_new = fmaxf(m, mt);
      const float mc = (m_new == kNegInf) ? 0.f : m_new * a.scale_log2;
      const float alpha = fast_exp2(m * a.scale_log2 - mc);
      m = m_new;
      // P^T (bf16) in the B-operand layout of chunk c: keys 16c + 8(e/4) + 4h + e%4
      bf16x8_t pb[4];
      float rs = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t pw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = fast_exp2(fmaf(s[c >> 1][8 * (c & 1) + e], a.scale_log2, -mc));
          const float p1 = fast_exp2(fmaf(s[c >> 1][8 * (c & 1) + e + 1], a.scale_log2, -mc));
          rs += p0 + p1;
          pw[e >> 1] = pack_bf16x2(p0, p1);
        }
        pb[c] = as_bf16x8((u32x4_t){pw[0], pw[1], pw[2], pw[3]});
      }
      l = l * alpha + rs;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      __syncthreads();  // V^T tile complete
      // O^T += V^T P^T: A operand row dv = 32db + l32, keys 16c + 4h + {0..3} and 16c + 8 + 4h + {0..3}
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint16_t* vrow = &Vt[(32 * db + l32) * VP + 16 * c + 4 * h];
          u32x2_t x0 = *(const u32x2_t*)vrow;
          u32x2_t x1 = *(const u32x2_t*)(vrow + 8);
          bf16x8_t va = as_bf16x8((u32x4_t){x0[0], x0[1], x1[0], x1[1]});
          o[db] = mfma32x32x16(va, pb[c], o[db]);
        }
      }
      ++kept;
    }
    if (mrow && t == 0) mrow[j] = keep ? 1 : 0;
  }
  if (mrow) {
    for (int j = J + t; j < a.nkt; j += NT) mrow[j] = 2;
  }

  // epilogue: this lane and lane ^ 32 hold partial sums of the same row
  const float lt = sum_with_lane_xor32(l);
  if (valid) {
    const float inv = 1.f / lt;
    const int64_t ob = b * a.os0 + hq * a.os1 + (int64_t)row * a.os2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        store_out4(a.out, ob + 32 * db + 8 * qd + 4 * h, a.out_f32, o[db][4 * qd] * inv,
                   o[db][4 * qd + 1] * inv, o[db][4 * qd + 2] * inv, o[db][4 * qd + 3] * inv);
    if (a.lse && h == 0) a.lse[(int64_t)bh * a.Nq + row] = m * a.scale + logf(lt);
  }
  if (a.stats && t == 0) {
    atomicAdd((unsigned long long*)&a.stats[2 * bh], (unsigned long long)J);
    atomicAdd((unsigned long long*)&a.stats[2 * bh + 1], (unsigned long long)kept);
  }
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  const int64_t nblocks = (int64_t)a.B * a.Hq * a.nqt;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)nblocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace blasst
