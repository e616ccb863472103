// Full non-causal attention of the H3 DiT block on gfx950 MFMA ([RV] README: the first public
// release uses full attention over the whole joint token sequence).
//
// One workgroup = 4 waves = 128 queries of one head (two workgroups per CU); each wave owns 32
// queries and walks all keys in blocks of 64 with an online softmax in the exp2 domain (the
// reference max is raised only when it would be exceeded by more than 2^8, so the output is
// rarely rescaled; all query tiles of a head share one XCD's L2).  Scores are computed
// transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16 with keys as rows), so each lane holds
// one query column: the row max and row sum are 16 lane-local values plus one exchange with
// the other half-wave, and the rescale of the output is a per-lane scalar.  O^T = V^T P^T
// reuses the score registers as the B operand; the key order inside a 16-key step is the
// score layout's (4 keys from each 8-key half), and V^T is stored with keys permuted inside
// each 16-key group (vt_pos) so that those 8 keys are adjacent: one 16-byte LDS read per step.
// K and V^T tiles go global -> LDS with buffer_load ... lds, double-buffered; the 16-byte
// chunks of a row are XOR-swizzled so that the 16 lanes of an LDS read phase (16 rows, one
// chunk) cover all 64 banks: c ^ (r & 15) for 256-byte rows, c ^ ((r >> 1) & 7) for 128.
// The key blocks are software-pipelined: the score MFMAs of block j+1 are interleaved with the
// exponentials of block j, and block j's O^T MFMAs with its row sums and block j+1's max, so
// that the matrix pipe and the VALU work on different blocks.  Each MFMA of the pipelined
// steps sits in a scheduling region of its own with the LDS fragment of the MFMA two places
// later read before it: left to itself, the scheduler read each V^T fragment just before its
// MFMA and waited for it there.  Values past the last key are
// cleared in the V^T fragments of the last block (the rows' padding may hold anything).
#include "common.hpp"

namespace h3 {

constexpr int ANW = 4;             // waves per workgroup
constexpr int AQ = 32 * ANW;       // queries per workgroup
constexpr int AKV = 64;            // keys per block
constexpr int ATHREADS = 64 * ANW;

template <int HD>
struct AttCfg {
  static constexpr int KROW = HD * 2;          // bytes per K row
  static constexpr int KBYTES = AKV * KROW;    // K tile
  static constexpr int VROW = AKV * 2;         // bytes per V^T row (64 keys)
  static constexpr int VBYTES = HD * VROW;     // V^T tile
  static constexpr int STAGE = KBYTES + VBYTES;
};

// three-input max (the compiler forms v_max3_f32)
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// max and sum of v over lanes l and l ^ 32 (the two half-waves), in every lane: one
// v_permlane32_swap, no LDS round trip.  The swap leaves lanes 0..31 of v in both halves of
// the first result and lanes 32..63 in both halves of the second.
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS slot of 16-byte chunk c in row r of a tile whose rows are `chunks` chunks long
__device__ __forceinline__ int att_slot(int c, int r, int chunks) {
  return chunks >= 16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

// Global -> LDS copies of one key block, 16 bytes per lane and instruction.  The buffer
// resource starts at the block (its range ends with the tensor, so rows past the end read as
// 0); the lane's offset inside the block is the same for every instruction of a wave up to a
// uniform stride, since the swizzle depends only on row bits that the stride leaves alone.
//
// K: AKV rows of HD*2 bytes (HD/8 chunks), 1024/KROW rows per instruction.  Lane offset
// of the wave's first row (wid) and of its own chunk:
template <int HD>
__device__ __forceinline__ uint32_t att_lane_k(int wid, int lane) {
  using C = AttCfg<HD>;
  constexpr int KCH = HD / 8, KRPI = 1024 / C::KROW;
  const int row = wid * KRPI + lane / KCH;
  return (uint32_t)(row * C::KROW + (att_slot(lane % KCH, row, KCH) << 4));
}
template <int HD>
__device__ __forceinline__ void att_load_k(const uint16_t *k, uint32_t k_bytes, uint8_t *dst, int64_t first_row,
                                           int wid, uint32_t lane_off) {
  using C = AttCfg<HD>;
  constexpr int KRPI = 1024 / C::KROW;
  const int64_t at = first_row * C::KROW;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(k + first_row * HD, k_bytes - (uint32_t)at);
#pragma unroll
  for (int i = 0; i < AKV / (KRPI * ANW); i++)
    buffer_load_lds16(rs, (lds_void *)(dst + (i * ANW + wid) * 1024), lane_off + (uint32_t)(i * ANW * 1024));
}
// V^T: HD rows of AKV keys = 128 bytes (8 chunks), 8 rows per instruction; rows are ldv
// elements apart
__device__ __forceinline__ uint32_t att_lane_v(int wid, int lane, int ldv) {
  const int row = wid * 8 + (lane >> 3);
  return (uint32_t)row * (uint32_t)ldv * 2u + (uint32_t)(att_slot(lane & 7, row, 8) << 4);
}
template <int HD>
__device__ __forceinline__ void att_load_v(const uint16_t *vt, uint32_t v_bytes, uint8_t *dst, int64_t first_elem,
                                           int ldv, int wid, uint32_t lane_off) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(vt + first_elem, v_bytes - (uint32_t)(first_elem * 2));
#pragma unroll
  for (int i = 0; i < HD / (8 * ANW); i++)
    buffer_load_lds16(rs, (lds_void *)(dst + (i * ANW + wid) * 1024), lane_off + (uint32_t)(i * ANW * 8 * ldv * 2));
}

// q and o may be the same buffer (the output written over the queries): neither is marked
// __restrict__.  Every Q load of a wave precedes its first O store, and waves read and write
// only their own query rows.
template <int HD>
__global__ __launch_bounds__(ATHREADS, 2) void k_attention(const uint16_t *q, const uint16_t *__restrict__ k,
                                                           const uint16_t *__restrict__ vt, uint16_t *o, int64_t N,
                                                           int ldv, int heads, float *row_max, float *row_sum) {
  using C = AttCfg<HD>;
  constexpr int KS = HD / 16;   // 16-dim steps of the score product
  constexpr int DT = HD / 32;   // 32-dim output tiles
  // LDS fragments are read two MFMAs ahead of their use in both products (deeper lookahead
  // measured no faster)
  constexpr int KD = 2, VD = 2;
  // two K and two V^T buffers as separate objects, so that the compiler sees that a prefetch
  // into one never aliases the reads of another
  __shared__ __attribute__((aligned(16))) uint8_t kbuf0[C::KBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t kbuf1[C::KBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vbuf0[C::VBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vbuf1[C::VBYTES];

  // Workgroups are dealt round-robin to the 8 XCDs in launch order.  When the head count
  // allows, all query tiles of one head go to the same XCD, so that its K and V^T are fetched
  // into one L2 instead of eight.
  const int QT = (int)gridDim.x;
  int h = blockIdx.y, qt = blockIdx.x;
  if ((heads & 7) == 0) {
    const int b = (int)blockIdx.y * QT + (int)blockIdx.x;
    const int j = b >> 3;
    h = (b & 7) + 8 * (j / QT);
    qt = j % QT;
  }
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform in the wave
  const int hsel = lane >> 5, l32 = lane & 31;
  const int64_t q0 = (int64_t)qt * AQ + wid * 32;
  const int64_t qrow = q0 + l32;
  const int64_t head_rows = (int64_t)h * N;
  const int64_t vfirst = (int64_t)h * HD * ldv;   // first element of the head's V^T rows

  const uint32_t k_bytes = (uint32_t)((int64_t)heads * N * HD * 2);
  const uint32_t v_bytes = (uint32_t)((int64_t)heads * HD * ldv * 2);
  const uint32_t lane_k = att_lane_k<HD>(wid, lane), lane_v = att_lane_v(wid, lane, ldv);
  auto load_k = [&](uint8_t *dst, int kb) { att_load_k<HD>(k, k_bytes, dst, head_rows + (int64_t)kb * AKV, wid, lane_k); };
  auto load_v = [&](uint8_t *dst, int kb) { att_load_v<HD>(vt, v_bytes, dst, vfirst + (int64_t)kb * AKV, ldv, wid, lane_v); };

  const int nkb = (int)((N + AKV - 1) / AKV);
  const int last_valid = (int)(N - (int64_t)(nkb - 1) * AKV);   // keys in the last block, 1..AKV
  load_k(kbuf0, 0);
  load_v(vbuf0, 0);

  // Q fragments (B operand: column = query, 8 dims per lane and step), kept in registers
  u32x4 qf[KS];
  {
    const int64_t qr = qrow < N ? qrow : N - 1;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(q + (head_rows + qr) * HD);
#pragma unroll
    for (int s = 0; s < KS; s++) qf[s] = src[2 * s + hsel];
  }
  const float c2 = (1.0f / sqrtf((float)HD)) * 1.4426950408889634f;  // score scale in log2 units

  f32x16 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; t++) acc[t] = f32x16{0};
  // Lazy rescaling: probabilities are taken relative to a reference m_ref (raw score units)
  // that is raised only when some lane's block max exceeds it by more than 2^8 in the exp2
  // domain, so p <= 256 and most blocks skip the output rescale.  m_true tracks the true max
  // for the row statistics; l_run sums 2^((s - m_ref) c2) over the lane's own keys (the two
  // half-waves' sums are added at the end).
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.0f;

  // S^T = K Q^T for the 64 keys of one block: two 32-key tiles (lane = one query; register r
  // of tile t holds key 32t + 8(r/4) + 4 hsel + r%4)
  auto scores = [&](const uint8_t *kb_, f32x16 (&s)[2]) {
    s[0] = f32x16{0};
    s[1] = f32x16{0};
#pragma unroll
    for (int st = 0; st < KS; st++)
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int krow = t * 32 + l32;
        const u32x4 kf = *reinterpret_cast<const u32x4 *>(kb_ + krow * C::KROW + (att_slot(2 * st + hsel, krow, HD / 8) << 4));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qf[st]),
                                                       s[t], 0, 0, 0);
      }
  };
  // keys past the end (the last block only) get score -inf
  // (the lane's keys are 4 hsel + c for constants c: one comparison with lim per key)
  auto mask = [&](f32x16 (&s)[2]) {
    const int lim = last_valid - 4 * hsel;
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        if (t * 32 + 8 * (r / 4) + (r % 4) >= lim) s[t][r] = -INFINITY;
  };
  // block max on raw scores (the scale c2 > 0 keeps the order), over the lane's 32 keys and
  // the other half-wave's
  auto block_max = [&](const f32x16 (&s)[2]) {
    float mq[4];
#pragma unroll
    for (int u = 0; u < 4; u++) mq[u] = fmaxf(s[u >> 1][(u & 1) * 8], s[u >> 1][(u & 1) * 8 + 1]);
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        if ((r & 7) > 1) mq[t * 2 + (r >> 3)] = fmaxf(mq[t * 2 + (r >> 3)], s[t][r]);
    const float mb = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    return halves_max(mb);
  };
  // raise the reference (and rescale what was summed against the old one) only when a lane's
  // scores would exceed it by more than 2^8; the first block always does
  auto rebase = [&](float mb) {
    m_true = fmaxf(m_true, mb);
    if (__any((mb - m_ref) * c2 > 8.0f)) {
      const float m_new = fmaxf(m_ref, mb);
      const float corr = __builtin_amdgcn_exp2f((m_ref - m_new) * c2);   // 0 on the first block
      l_run *= corr;
#pragma unroll
      for (int t = 0; t < DT; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[t][r] *= corr;
      m_ref = m_new;
    }
  };
  // p = 2^(s c2 - m_ref c2), one fma and one exp2 per score, in place
  auto probs = [&](f32x16 (&s)[2]) {
    const float mc = m_ref * c2;
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) s[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c2, -mc));
  };
  // O^T += V^T P^T over four 16-key steps, and the row sum of P.  The key order inside a step is
  // the score layout's: keys 16ps+4h..+3 and 16ps+8+4h..+3 sit at positions 16ps+8h..+7 of the
  // V^T row, chunk 2ps+h.  In the last block, values of keys past the end (the row's padding,
  // which may hold anything, NaN included) are cleared in the fragment, so that their zero
  // weights give zero.
  auto pv = [&](const uint8_t *vb_, const f32x16 (&s)[2], bool tail) {
    float lq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ps = 0; ps < 4; ps++) {
      const int t = ps >> 1, rb = 8 * (ps & 1);
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; j++) pf[j] = (__bf16)s[t][rb + j];
      uint32_t keep[4] = {~0u, ~0u, ~0u, ~0u};
      if (tail) {
        const int lim = last_valid - 4 * hsel;
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const int c = 16 * ps + 8 * (w >> 1) + 2 * (w & 1);   // keys 4 hsel + c, + 1 of the word's halves
          keep[w] = (c < lim ? 0xFFFFu : 0u) | (c + 1 < lim ? 0xFFFF0000u : 0u);
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        const int row = dt * 32 + l32;
        u32x4 vf = *reinterpret_cast<const u32x4 *>(vb_ + row * C::VROW + (att_slot(2 * ps + hsel, row, 8) << 4));
        if (tail) {
#pragma unroll
          for (int w = 0; w < 4; w++) vf[w] &= keep[w];
        }
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf), pf, acc[dt], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; j++) lq[ps] += s[t][rb + j];
    }
    float ls = (lq[0] + lq[1]) + (lq[2] + lq[3]);
    l_run += ls;
  };

  // The steady-state phases below are written in the order the instructions should issue:
  // each MFMA is followed by its share of the VALU work of the other block, and each LDS
  // fragment is read one MFMA pair ahead of its use.
  auto kfrag = [&](const uint8_t *kb_, int st, int t) {
    const int krow = t * 32 + l32;
    return *reinterpret_cast<const u32x4 *>(kb_ + krow * C::KROW + (att_slot(2 * st + hsel, krow, HD / 8) << 4));
  };
  auto vfrag = [&](const uint8_t *vb_, int ps, int dt) {
    const int row = dt * 32 + l32;
    return *reinterpret_cast<const u32x4 *>(vb_ + row * C::VROW + (att_slot(2 * ps + hsel, row, 8) << 4));
  };
  // scores of the next block (sn) on MFMA, probabilities of the current one (sc) on VALU; each
  // MFMA in a scheduling region of its own with the K fragment KD MFMAs later read before it.
  // The first VD V^T fragments of the O^T update (vb_) are read during the last score MFMAs.
  constexpr int NK = 2 * KS, NV = 4 * DT;
  auto scores_probs = [&](const uint8_t *kb_, const uint8_t *vb_, f32x16 (&sn)[2], f32x16 (&sc)[2],
                          u32x4 (&fv)[VD]) {
    constexpr int PER = 32 / KS;   // probabilities per score step
    // The score phase (each MFMA followed by two exponentials of the other block) runs at
    // raised wave priority: on a SIMD shared with a wave in its O^T phase its instructions
    // issue first and the other wave's fill in (about 1% faster on one box)
    __builtin_amdgcn_s_setprio(1);
    const float mc = m_ref * c2;
    sn[0] = f32x16{0};
    sn[1] = f32x16{0};
    u32x4 fk[KD];
#pragma unroll
    for (int i = 0; i < KD; i++) fk[i] = kfrag(kb_, i >> 1, i & 1);
#pragma unroll
    for (int i = 0; i < NK; i++) {
      const int st = i >> 1, t = i & 1;
      u32x4 nk = fk[0];
      if (i + KD < NK) nk = kfrag(kb_, (i + KD) >> 1, (i + KD) & 1);
      if (i + VD >= NK) fv[i + VD - NK] = vfrag(vb_, (i + VD - NK) / DT, (i + VD - NK) % DT);
      sn[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fk[0]), __builtin_bit_cast(bf16x8, qf[st]),
                                                      sn[t], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < PER / 2; e++) {
        const int k = st * PER + t * (PER / 2) + e;
        sc[k >> 4][k & 15] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[k >> 4][k & 15], c2, -mc));
      }
#pragma unroll
      for (int r = 0; r + 1 < KD; r++) fk[r] = fk[r + 1];
      fk[KD - 1] = nk;
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // O^T update with the current block's probabilities on MFMA; their row sum and the next
  // block's max on VALU.  Returns the next block's max (both half-waves).  The MFMAs go in
  // (ps, dt) order, each in a scheduling region of its own, with the V^T fragment of the MFMA
  // VD places later read before it (fv: the first VD, read by the caller), and the
  // probabilities of step ps+1 converted during step ps.
  auto pv_max = [&](const uint8_t *vb_, u32x4 (&fv)[VD], const f32x16 (&sc)[2], const f32x16 (&sn)[2]) {
    float lq[4], mq[4];
    bf16x8 pf, pn;
#pragma unroll
    for (int j = 0; j < 8; j++) pf[j] = (__bf16)sc[0][j];
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int ps = i / DT, dt = i % DT;
      const int t = ps >> 1, rb = 8 * (ps & 1);
      u32x4 nv = fv[0];
      if (i + VD < NV) nv = vfrag(vb_, (i + VD) / DT, (i + VD) % DT);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fv[0]), pf, acc[dt], 0, 0, 0);
      if (dt == 0) {
        lq[ps] = sc[t][rb];
#pragma unroll
        for (int j = 1; j < 8; j++) lq[ps] += sc[t][rb + j];
      }
      if (dt == 1) {
        mq[ps] = max3f(sn[t][rb], sn[t][rb + 1], sn[t][rb + 2]);
        mq[ps] = max3f(mq[ps], sn[t][rb + 3], sn[t][rb + 4]);
        mq[ps] = max3f(mq[ps], sn[t][rb + 5], sn[t][rb + 6]);
        mq[ps] = fmaxf(mq[ps], sn[t][rb + 7]);
      }
      if (dt == DT / 2 && ps + 1 < 4) {
        const int t1 = (ps + 1) >> 1, rb1 = 8 * ((ps + 1) & 1);
#pragma unroll
        for (int j = 0; j < 8; j++) pn[j] = (__bf16)sc[t1][rb1 + j];
      }
      if (dt == DT - 1) pf = pn;
#pragma unroll
      for (int r = 0; r + 1 < VD; r++) fv[r] = fv[r + 1];
      fv[VD - 1] = nv;
      __builtin_amdgcn_sched_barrier(0);
    }
    float ls = (lq[0] + lq[1]) + (lq[2] + lq[3]);
    l_run += ls;
    const float mb = max3f(mq[0], mq[1], fmaxf(mq[2], mq[3]));
    return halves_max(mb);
  };

  // Software pipeline over the key blocks: while the MFMAs of block j+1's scores run, the VALU
  // turns block j's scores into probabilities; while the MFMAs of block j's O^T update run, it
  // sums block j's probabilities and takes block j+1's max.  K runs one block ahead of V^T:
  // during step j, K(j+2) is fetched into the buffer K(j) used and V^T(j+1) into the one of
  // V^T(j-1); the barrier at the start of each step orders both after the last reads of what
  // they overwrite.
  f32x16 sa[2], sb[2];
  if (nkb > 1) load_k(kbuf1, 1);
  wait_vmem();
  __syncthreads();
  scores(kbuf0, sa);
  if (nkb == 1 && last_valid < AKV) mask(sa);
  rebase(block_max(sa));

  // step j: K(j+1) sits in kn, V^T(j) in vc; kc (K(j)'s buffer) receives K(j+2), vn V^T(j+1)
  // (interior: j + 3 < nkb is known, so that neither test below branches)
  auto step = [&](bool interior, int j, uint8_t *kc, const uint8_t *kn, uint8_t *vc, uint8_t *vn, f32x16 (&sc)[2],
                  f32x16 (&sn)[2]) {
    wait_vmem();
    __syncthreads();
    if (interior || j + 2 < nkb) load_k(kc, j + 2);
    load_v(vn, j + 1);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 fv[VD];
    scores_probs(kn, vc, sn, sc, fv);
    __builtin_amdgcn_sched_barrier(0);
    if (!interior && j + 2 == nkb && last_valid < AKV) mask(sn);
    __builtin_amdgcn_sched_barrier(0);
    const float mb = pv_max(vc, fv, sc, sn);
    rebase(mb);
  };
  // last step: V^T(nkb-1) in vc, its probabilities from sc
  auto last = [&](const uint8_t *vc, f32x16 (&sc)[2]) {
    wait_vmem();
    __syncthreads();
    probs(sc);
    pv(vc, sc, true);
  };
  // Steps run in pairs so that every buffer is named statically; the pairs whose steps are all
  // interior loop, the last one or two steps and the last block follow.
  int j = 0;
  for (; j + 3 < nkb; j += 2) {
    step(true, j, kbuf0, kbuf1, vbuf0, vbuf1, sa, sb);
    step(true, j + 1, kbuf1, kbuf0, vbuf1, vbuf0, sb, sa);
  }
  // (one or two steps left, or none; the last block's probabilities are brought into sa so
  // that one copy of the last step serves every count)
  const uint8_t *vlast = vbuf0;
  if (j + 1 < nkb) {
    step(false, j, kbuf0, kbuf1, vbuf0, vbuf1, sa, sb);
    if (j + 2 < nkb) {
      step(false, j + 1, kbuf1, kbuf0, vbuf1, vbuf0, sb, sa);
    } else {
      sa[0] = sb[0];
      sa[1] = sb[1];
      vlast = vbuf1;
    }
  }
  last(vlast, sa);

  // O[h][q][dim] = O^T / l; lane holds dims dt*32 + 8(r/4) + 4 hsel + r%4 of query qrow
  l_run = halves_sum(l_run);
  if (qrow < N) {
    const float inv = 1.0f / l_run;
    uint16_t *dst = o + (head_rows + qrow) * HD;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int dim = dt * 32 + 8 * g + 4 * hsel;
        uint2 v;
        v.x = pack_bf2(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv);
        v.y = pack_bf2(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv);
        *reinterpret_cast<uint2 *>(dst + dim) = v;
      }
    if (row_max && hsel == 0) {
      row_max[head_rows + qrow] = m_true * (1.0f / sqrtf((float)HD));
      row_sum[head_rows + qrow] = l_run * __builtin_amdgcn_exp2f((m_ref - m_true) * c2);
    }
  }
}

hipError_t launch_attention(int heads, int64_t n, int hd, const uint16_t *q, const uint16_t *k, const uint16_t *vt,
                            uint16_t *o, float *row_max, float *row_sum, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int ldv = (int)vt_pitch(n);
  dim3 grid((unsigned)((n + AQ - 1) / AQ), (unsigned)heads);
  if (hd == 128)
    k_attention<128><<<grid, ATHREADS, 0, st>>>(q, k, vt, o, n, ldv, heads, row_max, row_sum);
  else
    k_attention<64><<<grid, ATHREADS, 0, st>>>(q, k, vt, o, n, ldv, heads, row_max, row_sum);
  return hipGetLastError();
}

}  // namespace h3
