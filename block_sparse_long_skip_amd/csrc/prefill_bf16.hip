// bf16 skip-softmax prefill, d_qk = d_v = 128, 128-row query tiles, 64-key
// tiles, on gfx950 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Method: BLASST post (seeallochnaya, "BLASST: Dynamic BLocked Attention
// Sparsity via Softmax Thresholding"): key tiles in increasing order (paragraph
// "В чём идея"), online max with rescale (paragraph on FlashAttention 1), a
// tile dropped whole when its max is far below the running max and its V never
// read (paragraph beginning "BLASST предлагает"), tile 0 always processed
// (first figure). The drop test is one scalar threshold on the running-max
// statistics (digg thread "BLASST wins Best Paper at MLSys 2026"). The lazy
// rescale below follows the FlashAttention 4 idea the post describes (the
// paragraph on FlashAttention 4): partial sums are rescaled only when the
// running max has grown enough to threaten precision, which keeps the result
// exact; the drop decision always uses the exact running max.
//
// Layout. One workgroup of 4 waves per (batch, query head, query tile); wave w
// owns query rows [32w, 32w+32). Scores are computed transposed,
// S^T = K Q^T, so the MFMA result puts one query row in each lane column:
// lane l holds row 32w + (l & 31) and 32 of the tile's 64 keys (lane l ^ 32
// holds the other 32). Row max and row sum stay in-lane plus one lane swap.
// The output is accumulated transposed too, O^T = V^T P^T, so a rescale is a
// per-lane scalar. P^T feeds the second MFMA straight from the first MFMA's
// accumulators (the key order inside one MFMA's contraction is permuted to
// match the accumulator layout; the same permutation is applied to V^T, so the
// sum is unchanged). V^T comes from a row-major V tile through the gfx950
// transposing LDS read (ds_read_b64_tr_b16).
//
// Pipeline (one barrier per key tile). At the top of iteration j the scores
// S_j are in registers, the decision for tile j is known, the V_j loads into
// LDS are in flight (kept tiles only) and K_{j+1} is in LDS. The iteration
// issues the K_{j+2} loads, computes S_{j+1} on MFMA while the VALU turns S_j
// into P_j, votes on tile j+1, waits for its own loads, meets the barrier,
// issues the V_{j+1} loads only if tile j+1 is kept, and then runs
// O^T += V_j^T P_j^T.
// So V is fetched only after the vote, and its latency hides behind a whole
// tile of work. The vote for tile j+1 needs the running max before it, which
// for lambda <= 1 is the plain prefix max of the row maxima (a dropped tile
// cannot raise it), so it does not wait for the softmax of tile j.
//
// LDS: K and V tiles double-buffered, 64 rows x 256 B each, unpadded, with the
// 16-byte chunk index XOR-swizzled by the row so that both the K operand reads
// (16 rows, one chunk) and the transposing V reads (4 rows, 2 chunks) hit
// distinct banks. Tiles travel global -> LDS with buffer_load_dwordx4 ... lds
// (no register staging): a buffer resource per tile (uniform base and range),
// a per-lane 32-bit offset fixed for the whole loop, and no vector ALU work
// per copy. LDS reads are a per-lane base plus immediate offsets.
//
// Block-sparse mode (the MASKED instance): attention is restricted to a
// caller-given set of (query tile, key tile) blocks, as in the final stage of
// block-sparse prefill methods, which compute ordinary softmax attention inside
// the selected blocks (CRISP summary on rit.work, section "Что сделали"). The
// workgroup first lists its row of the set in LDS, in increasing key order;
// the pipeline above then walks that list instead of [0, J), so tiles outside
// the set cost nothing and the skip rule runs over the set's tiles only.
#include <type_traits>

#include "common.hpp"

namespace blasst {

namespace {
constexpr int D = 128;
constexpr int BR = 128;
constexpr int BC = 64;
constexpr int NT = 256;
constexpr int TILE_BYTES = BC * D * 2;  // 16 KB
constexpr float kLazyRescaleLog2 = 8.f;  // rescale once the max grows by 2^8
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: 32-bit data format, raw access

// XOR applied to the 16-byte chunk index of tile row `row`
__device__ __forceinline__ int swz_f(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
// byte offset of (row, 16-byte chunk c) inside a 64 x 256 B tile
__device__ __forceinline__ int swz(int row, int c) { return row * 256 + ((c ^ swz_f(row)) << 4); }

struct RowState {
  float m_prefix;  // exact running max (raw q.k units) of this lane's row, -inf before tile 0
  float m_acc;     // reference max of the accumulators (<= m_prefix, within 2^8 in exp2 units)
  float l;         // this lane's partial row sum (half of the row's keys)
};

}  // namespace

// MASKED: block-sparse mode. The query tile visits only the key tiles of its
// row of the block set, in increasing order, from a list built in LDS.
template <bool MASKED>
__global__ void __launch_bounds__(NT, 2) prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char Ks[2][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char Vs[2][TILE_BYTES];
  __shared__ int votes[2][4];
  __shared__ uint16_t tlist[MASKED ? kPrefillMaxSetTiles : 1];
  __shared__ int wcount[4];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // block -> (query tile, batch, head). A unit of work is a (batch, KV head,
  // query tile) triple; units go heaviest query tiles first. The G query heads
  // of a unit read the same K/V tiles in the same order, so they take G
  // consecutive slots of one XCD (the hardware deals blocks to the 8 XCDs
  // round-robin: block x runs on XCD x % 8, as its slot x / 8 there) and run
  // together out of that XCD's L2. Units are dealt to the XCDs round-robin;
  // blocks past the last unit (when the unit count is not a multiple of 8)
  // return at once.
  const int G = a.Hq / a.Hkv;
  const int ngrp = a.B * a.Hkv;
  const int slot = (int)(blockIdx.x >> 3);
  const int64_t u = (int64_t)(slot / G) * 8 + (blockIdx.x & 7);
  if (u >= (int64_t)ngrp * a.nqt) return;
  const int i = a.nqt - 1 - (int)(u / ngrp);
  const int grp = (int)(u % ngrp);
  const int b = grp / a.Hkv, kvh = grp % a.Hkv;
  const int hq = kvh * G + slot % G;
  const int bh = b * a.Hq + hq;

  const uint16_t* qp = (const uint16_t*)a.q + b * a.qs0 + hq * a.qs1;
  const char* kp = (const char*)((const uint16_t*)a.k + b * a.ks0 + kvh * a.ks1);
  const char* vp = (const char*)((const uint16_t*)a.v + b * a.vs0 + kvh * a.vs1);

  const int row = i * BR + 32 * w + l32;  // this lane's query row
  const bool valid = row < a.Nq;
  const int qpos = row + (a.Nk - a.Nq);
  const int last_row = min(i * BR + BR - 1, a.Nq - 1);
  const int first_pos = i * BR + (a.Nk - a.Nq);  // key position of the tile's first row
  const int J = a.causal ? min(a.nkt, (last_row + a.Nk - a.Nq) / BC + 1) : a.nkt;
  const float c2 = a.scale_log2;

  // Q^T as the B operand: lane supplies Q[row][16kk + 8h .. +7]
  bf16x8_t qb[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (valid) v = load16(qp + (int64_t)row * a.qs2 + 16 * kk + 8 * h);
    qb[kk] = as_bf16x8(v);
  }

  // ---- per-lane addresses, computed once
  // Tile loads: wave w fills rows 16w..16w+15, 4 rows per instruction; lane l
  // lands at (instruction base + 16 l) = row 4r + l/16, physical chunk l%16, so
  // it fetches the logical chunk the swizzle maps there.
  const int sub = lane >> 4, pch = lane & 15;
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int trow = 16 * w + 4 * r + sub;
    const int ch = pch ^ swz_f(trow);
    koff[r] = (uint32_t)(((int64_t)trow * a.ks2 + ch * 8) * 2);
    voff[r] = (uint32_t)(((int64_t)trow * a.vs2 + ch * 8) * 2);
  }
  // One tile into LDS through a buffer resource whose range ends at the last
  // key of the sequence: the hardware returns zeros for rows past it (their
  // scores are masked to -inf, and their values meet p = 0). The per-lane
  // offsets above do not depend on the tile; base, range and LDS address are
  // uniform.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto tile_to_lds = [&](char* tile, const char* base, const uint32_t (&off)[4], int64_t stride,
                         int c0) {
    const uint64_t tb = (uint64_t)(base + (int64_t)c0 * stride * 2);
    const uint64_t ub = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(tb >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tb);
    const int rows = __builtin_amdgcn_readfirstlane(min(a.Nk - c0, BC));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)ub, (short)0, (int)((uint32_t)rows * (uint32_t)(stride * 2)), kBufferFlags);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(tile + (16 * wu + 4 * r) * 256), 16, off[r],
          0, 0, 0);
  };
  // K operand reads: key row 32kb + l32, chunk 2kk + h (kb = 1 is +8192 bytes)
  int kro[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kro[kk] = swz(l32, 2 * kk + h);
  // V^T operand reads (transposing): lane group g16 = lane/16 reads keys
  // 16c + 4h + jj/4 and +8 (key chunk c is +4096 bytes), features dv0..dv0+3
  const int g16 = lane >> 4, jj = lane & 15;
  int vro[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int dv0 = 32 * db + 16 * (g16 & 1) + 4 * (jj & 3);
    const int r0 = 4 * h + (jj >> 2);
    vro[db][0] = swz(r0, dv0 >> 3) + ((dv0 & 7) << 1);
    vro[db][1] = swz(r0 + 8, dv0 >> 3) + ((dv0 & 7) << 1);
  }

  // S^T for one key tile from LDS: the two 32-key blocks are independent MFMA
  // chains, interleaved, with each step's two K operands read two steps ahead
  // (a three-deep register ring) so the LDS latency is covered by four MFMAs
  auto scores = [&](const char* kt, f32x16_t (&s)[2]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[0][r] = s[1][r] = 0.f;
    u32x4_t ka[3], kb[3];
    ka[0] = *(const u32x4_t*)(kt + kro[0]);
    kb[0] = *(const u32x4_t*)(kt + 8192 + kro[0]);
    ka[1] = *(const u32x4_t*)(kt + kro[1]);
    kb[1] = *(const u32x4_t*)(kt + 8192 + kro[1]);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (kk + 2 < D / 16) {
        ka[(kk + 2) % 3] = *(const u32x4_t*)(kt + kro[kk + 2]);
        kb[(kk + 2) % 3] = *(const u32x4_t*)(kt + 8192 + kro[kk + 2]);
      }
      s[0] = mfma32x32x16(as_bf16x8(ka[kk % 3]), qb[kk], s[0]);
      s[1] = mfma32x32x16(as_bf16x8(kb[kk % 3]), qb[kk], s[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P_j (bf16, B-operand layout of chunk c: keys 16c + 8(e/4) + 4h + e%4)
  // from S_j: the four values of step x = 4c' + ... live in pw; the row sum
  // adds the fp32 values so lse stays fp32-accurate
  auto probs_step = [&](const f32x16_t (&s)[2], float mc, int x, uint32_t (&pw)[4][4],
                        float& ls0, float& ls1) {
    const int c = x >> 1, e0 = 4 * (x & 1);
    const float p0 = fast_exp2(fmaf(s[c >> 1][8 * (c & 1) + e0], c2, -mc));
    const float p1 = fast_exp2(fmaf(s[c >> 1][8 * (c & 1) + e0 + 1], c2, -mc));
    const float p2 = fast_exp2(fmaf(s[c >> 1][8 * (c & 1) + e0 + 2], c2, -mc));
    const float p3 = fast_exp2(fmaf(s[c >> 1][8 * (c & 1) + e0 + 3], c2, -mc));
    pw[c][2 * (x & 1)] = pack_bf16x2(p0, p1);
    pw[c][2 * (x & 1) + 1] = pack_bf16x2(p2, p3);
    ls0 += p0 + p2;
    ls1 += p1 + p3;
  };
  // S_{j+1} on MFMA and P_j on the VALU, interleaved in program order: each of
  // the 8 steps issues the two K-operand reads of the step after next, two
  // MFMAs (one per 32-key block) and a quarter-chunk of P_j; the scheduling
  // fence keeps that order, so a wave fills its own MFMA dependency stalls
  // with softmax work
  auto scores_and_probs = [&](const char* kt, f32x16_t (&sn)[2], const f32x16_t (&s)[2],
                              float mc, bf16x8_t (&pb)[4], float& lsum) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sn[0][r] = sn[1][r] = 0.f;
    uint32_t pw[4][4];
    float ls0 = 0.f, ls1 = 0.f;
    u32x4_t ka[3], kb[3];
    ka[0] = *(const u32x4_t*)(kt + kro[0]);
    kb[0] = *(const u32x4_t*)(kt + 8192 + kro[0]);
    ka[1] = *(const u32x4_t*)(kt + kro[1]);
    kb[1] = *(const u32x4_t*)(kt + 8192 + kro[1]);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (kk + 2 < D / 16) {
        ka[(kk + 2) % 3] = *(const u32x4_t*)(kt + kro[kk + 2]);
        kb[(kk + 2) % 3] = *(const u32x4_t*)(kt + 8192 + kro[kk + 2]);
      }
      sn[0] = mfma32x32x16(as_bf16x8(ka[kk % 3]), qb[kk], sn[0]);
      sn[1] = mfma32x32x16(as_bf16x8(kb[kk % 3]), qb[kk], sn[1]);
      probs_step(s, mc, kk, pw, ls0, ls1);
      // consume this step's results here so they are not sunk past the MFMAs
      asm volatile("" ::"v"(pw[kk >> 1][2 * (kk & 1)]), "v"(pw[kk >> 1][2 * (kk & 1) + 1]),
                   "v"(ls0), "v"(ls1));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) pb[c] = as_bf16x8((u32x4_t){pw[c][0], pw[c][1], pw[c][2], pw[c][3]});
    lsum += ls0 + ls1;
  };
  // tiles that cross the end of the sequence or (causal) this tile's diagonal
  auto tile_needs_mask = [&](int c0) {
    return (c0 + BC > a.Nk) || (a.causal && c0 + BC - 1 > first_pos);
  };
  // masks keys past Nk and (causal) keys after this lane's row
  auto mask_scores = [&](int c0, f32x16_t (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int col = c0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
        if (col >= a.Nk || (a.causal && col > qpos)) s[kb][r] = kNegInf;
      }
  };
  auto rowmax = [&](const f32x16_t (&s)[2]) {
    float m0 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
    float m1 = fmaxf(fmaxf(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      m0 = fmaxf(fmaxf(m0, s[0][r]), s[0][r + 1]);
      m1 = fmaxf(fmaxf(m1, s[1][r]), s[1][r + 1]);
    }
    m0 = fmaxf(fmaxf(m0, s[0][15]), m1);
    m0 = fmaxf(m0, s[1][15]);
    return max_with_lane_xor32(m0);
  };
  // this lane's vote: keep unless its row's gap is below the threshold
  auto lane_vote = [&](float mt, float m_before) {
    float gap;
    if (mt == kNegInf) gap = kNegInf;
    else if (m_before == kNegInf) gap = __builtin_inff();
    else gap = mt - m_before;
    return valid && !(gap < a.thr_raw);
  };

  f32x16_t o[4];  // O^T[dv = 32db + 8(r/4) + 4h + r%4][row], relative to st.m_acc
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  RowState st = {kNegInf, kNegInf, 0.f};
  int kept = 0;
  uint8_t* mrow = a.mask ? a.mask + ((int64_t)bh * a.nqt + i) * a.nkt : nullptr;

  // The n key tiles this query tile visits: [0, J), or in block-sparse mode
  // the set's tiles among them, listed in increasing order. The list is built
  // from per-thread runs of consecutive tiles and a prefix sum of the run
  // counts; blocks outside the set get mask 2 here.
  int n = J;
  if constexpr (MASKED) {
    const uint8_t* sel = a.block_mask + b * a.bms0 + hq * a.bms1 + (int64_t)i * a.bms2;
    const int per = (J + NT - 1) / NT;
    const int x0 = min(t * per, J), x1 = min(x0 + per, J);
    int cnt = 0;
    for (int x = x0; x < x1; ++x) cnt += sel[x] != 0;
    int incl = cnt;  // inclusive prefix sum over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wcount[w] = incl;
    __syncthreads();
    int pos = incl - cnt;
    for (int ww = 0; ww < w; ++ww) pos += wcount[ww];
    n = __builtin_amdgcn_readfirstlane(wcount[0] + wcount[1] + wcount[2] + wcount[3]);
    for (int x = x0; x < x1; ++x) {
      if (sel[x]) tlist[pos++] = (uint16_t)x;
      else if (mrow) mrow[x] = 2;
    }
    if (mrow)
      for (int x = J + t; x < a.nkt; x += NT) mrow[x] = 2;
    __syncthreads();
  }
  // key-tile index of the x-th visited tile (uniform)
  auto tile_at = [&](int x) -> int {
    if constexpr (MASKED) return __builtin_amdgcn_readfirstlane((int)tlist[x]);
    else return x;
  };

  f32x16_t sA[2], sB[2];
  float mt = kNegInf;
  bool keep = true;
  int j = 0;
  // one key tile; P = j & 1 (compile-time), s = S_j, sn receives S_{j+1}
  auto step = [&](auto PAR, f32x16_t (&s)[2], f32x16_t (&sn)[2]) {
    constexpr int P = decltype(PAR)::value;
    const int c0 = tile_at(j) * BC;
    const bool has_next = j + 1 < n;
    const int cn = has_next ? tile_at(j + 1) * BC : 0;
    // (a) K_{j+2} straight into the buffer K_j used (every wave read it before
    //     the previous barrier)
    if (j + 2 < n) tile_to_lds(Ks[P], kp, koff, a.ks2, tile_at(j + 2) * BC);
    // (b, c) scores of tile j+1 (MFMA) and P_j (VALU)
    st.m_prefix = fmaxf(st.m_prefix, mt);  // running max through tile j
    bf16x8_t pb[4];
    if (keep) {
      // lazy rescale: move the accumulators' reference max only when the exact
      // max has grown by more than 2^8 (any lane of the wave), or on the first tile
      const bool grow = (st.m_prefix - st.m_acc) * c2 > kLazyRescaleLog2;
      if (__any(grow)) {
        // a row that has seen no key yet (block-sparse mode: its running max is
        // still -inf) keeps its empty sums as they are
        const float alpha =
            st.m_prefix == kNegInf ? 1.f : fast_exp2((st.m_acc - st.m_prefix) * c2);
        st.m_acc = st.m_prefix;
        st.l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
    }
    // (a row with no reference max yet has only -inf scores: p = 0 against 0)
    const float mc = st.m_acc == kNegInf ? 0.f : st.m_acc * c2;
    if (has_next && keep) {
      scores_and_probs(Ks[P ^ 1], sn, s, mc, pb, st.l);
    } else if (has_next) {
      scores(Ks[P ^ 1], sn);
    } else if (keep) {
      uint32_t pw[4][4];
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int x = 0; x < 8; ++x) probs_step(s, mc, x, pw, ls0, ls1);
#pragma unroll
      for (int c = 0; c < 4; ++c) pb[c] = as_bf16x8((u32x4_t){pw[c][0], pw[c][1], pw[c][2], pw[c][3]});
      st.l += ls0 + ls1;
    }
    if (has_next && tile_needs_mask(cn)) mask_scores(cn, sn);
    // (e) vote on tile j+1 against the running max through tile j
    float mtn = kNegInf;
    if (has_next) {
      mtn = rowmax(sn);
      const bool wave_keep = __any(lane_vote(mtn, st.m_prefix));
      if (lane == 0) votes[P ^ 1][w] = wave_keep ? 1 : 0;
    }
    // (f) V_j (issued after tile j's vote) and K_{j+2} have landed in LDS
    wait_vmem();
    __syncthreads();
    bool keep_next = false;
    if (has_next) {
      const int* vv = votes[P ^ 1];
      keep_next = (vv[0] | vv[1] | vv[2] | vv[3]) != 0;
      if (mrow && t == 0) mrow[cn / BC] = keep_next ? 1 : 0;
      // (h) V_{j+1} is fetched only for a kept tile, into the buffer V_{j-1}
      //     used (every wave finished reading it before this barrier)
      if (keep_next) tile_to_lds(Vs[P ^ 1], vp, voff, a.vs2, cn);
    }
    // (i) O^T += V_j^T P_j^T: per key chunk c, the 4 output blocks are
    //     independent MFMA chains; the next chunk's V^T reads are issued first
    if (keep) {
      const char* vt = Vs[P];
      u32x4_t va[4], vb[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2_t y0 = ds_read_tr(vt + vro[db][0]), y1 = ds_read_tr(vt + vro[db][1]);
        va[db] = (u32x4_t){y0[0], y0[1], y1[0], y1[1]};
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c + 1 < 4) {
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const u32x2_t y0 = ds_read_tr(vt + 4096 * (c + 1) + vro[db][0]);
            const u32x2_t y1 = ds_read_tr(vt + 4096 * (c + 1) + vro[db][1]);
            vb[db] = (u32x4_t){y0[0], y0[1], y1[0], y1[1]};
          }
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = mfma32x32x16(as_bf16x8(va[db]), pb[c], o[db]);
#pragma unroll
        for (int db = 0; db < 4; ++db) va[db] = vb[db];
      }
      // schedule: the first three MFMAs' V^T reads, then each MFMA followed by
      // the reads of the MFMA three places later (left alone, the scheduler
      // issues each read pair just one MFMA ahead of its use)
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int x = 0; x < 13; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      ++kept;
    }
    keep = keep_next;
    mt = mtn;
    ++j;
  };
  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
  if (n > 0) {
    // ---- prologue: K_0, K_1 and V_0 (the first visited tile is always kept)
    //      into LDS, then S_0
    const int c0 = tile_at(0) * BC;
    tile_to_lds(Ks[0], kp, koff, a.ks2, c0);
    if (n > 1) tile_to_lds(Ks[1], kp, koff, a.ks2, tile_at(1) * BC);
    tile_to_lds(Vs[0], vp, voff, a.vs2, c0);
    wait_vmem();
    __syncthreads();
    scores(Ks[0], sA);
    if (tile_needs_mask(c0)) mask_scores(c0, sA);
    mt = rowmax(sA);
    if (mrow && t == 0) mrow[c0 / BC] = 1;
    __syncthreads();  // every wave has read K_0 before it is overwritten
    while (j < n) {
      step(even, sA, sB);
      if (j >= n) break;
      step(odd, sB, sA);
    }
  }
  if (!MASKED && mrow) {
    for (int x = J + t; x < a.nkt; x += NT) mrow[x] = 2;
  }

  // epilogue: this lane and lane ^ 32 hold partial sums of the same row. In
  // block-sparse mode a row may see no key at all (its running max is still
  // -inf and its sums are not meaningful): it outputs zero and lse -inf.
  const float lt = sum_with_lane_xor32(st.l);
  if (valid) {
    const bool seen = !MASKED || st.m_prefix != kNegInf;
    const float inv = seen ? 1.f / lt : 0.f;
    auto ov = [&](float x) { return seen ? x * inv : 0.f; };
    const int64_t ob = b * a.os0 + hq * a.os1 + (int64_t)row * a.os2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        store_out4(a.out, ob + 32 * db + 8 * qd + 4 * h, a.out_f32, ov(o[db][4 * qd]),
                   ov(o[db][4 * qd + 1]), ov(o[db][4 * qd + 2]), ov(o[db][4 * qd + 3]));
    if (a.lse && h == 0)
      a.lse[(int64_t)bh * a.Nq + row] = seen ? st.m_acc * a.scale + logf(lt) : kNegInf;
  }
  if (a.stats && t == 0) {
    atomicAdd((unsigned long long*)&a.stats[2 * bh], (unsigned long long)n);
    atomicAdd((unsigned long long*)&a.stats[2 * bh + 1], (unsigned long long)kept);
  }
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  // whole rounds of 8 units (one per XCD), G blocks per unit
  const int64_t units = (int64_t)a.B * a.Hkv * a.nqt;
  const int64_t nblocks = (units + 7) / 8 * 8 * (a.Hq / a.Hkv);
  if (units == 0) return hipSuccess;
  if (a.block_mask)
    hipLaunchKernelGGL(prefill_bf16_kernel<true>, dim3((unsigned)nblocks), dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<false>, dim3((unsigned)nblocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace blasst
