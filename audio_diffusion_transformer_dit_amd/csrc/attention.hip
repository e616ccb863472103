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

// LDS slot of 16-byte chunk c in row r of a tile whose rows are `chunks` chunks long
__device__ __forceinline__ int att_slot(int c, int r, int chunks) {
  return chunks >= 16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

template <int HD>
__device__ __forceinline__ void att_load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint8_t *st,
                                         int64_t kbase_row, int64_t vbase_row, int ldv, int kb) {
  using C = AttCfg<HD>;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // K: rows of HD*2 bytes = HD/8 chunks; one instruction fills 1 KiB = 1024/KROW rows
  constexpr int KCH = HD / 8;
  constexpr int KRPI = 1024 / C::KROW;
  {
    const int rl = lane / KCH, slot = lane % KCH;
#pragma unroll
    for (int i = 0; i < AKV / (KRPI * ANW); i++) {
      const int rb = i * ANW + wid;
      const int row = rb * KRPI + rl;
      const int chunk = att_slot(slot, row, KCH);
      const uint32_t off = (uint32_t)(((kbase_row + (int64_t)kb * AKV + row) * HD + chunk * 8) * 2);
      buffer_load_lds16(rk, (lds_void *)(st + rb * 1024), off);
    }
  }
  // V^T: HD rows of 128 bytes (8 chunks), 8 rows per instruction
  {
    const int rl = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int i = 0; i < HD / (8 * ANW); i++) {
      const int rb = i * ANW + wid;
      const int row = rb * 8 + rl;
      const int chunk = att_slot(slot, row, 8);
      const uint32_t off = (uint32_t)((((vbase_row + row) * (int64_t)ldv) + (int64_t)kb * AKV + chunk * 8) * 2);
      buffer_load_lds16(rv, (lds_void *)(st + C::KBYTES + rb * 1024), off);
    }
  }
}

template <int HD>
// q and o may be the same buffer (the output written over the queries): neither is marked
// __restrict__.  Every Q load of a wave precedes its first O store, and waves read and write
// only their own query rows.
__global__ __launch_bounds__(ATHREADS, 2) void k_attention(const uint16_t *q, const uint16_t *__restrict__ k,
                                                           const uint16_t *__restrict__ vt, uint16_t *o, int64_t N,
                                                           int ldv, int heads, float *row_max, float *row_sum) {
  using C = AttCfg<HD>;
  constexpr int KS = HD / 16;   // 16-dim steps of the score product
  constexpr int DT = HD / 32;   // 32-dim output tiles
  // two LDS stages as separate objects, so that the compiler sees that the prefetch of one
  // never aliases the reads of the other (and does not wait for the prefetch before them)
  __shared__ __attribute__((aligned(16))) uint8_t stage0[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[C::STAGE];

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
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int hsel = lane >> 5, l32 = lane & 31;
  const int64_t q0 = (int64_t)qt * AQ + wid * 32;
  const int64_t qrow = q0 + l32;
  const int64_t head_rows = (int64_t)h * N;

  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k, (uint32_t)((int64_t)heads * N * HD * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vt, (uint32_t)((int64_t)heads * HD * ldv * 2));

  const int nkb = (int)((N + AKV - 1) / AKV);
  att_load<HD>(rk, rv, stage0, head_rows, (int64_t)h * HD, ldv, 0);

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
  // for the row statistics; l_run sums 2^((s - m_ref) c2).
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.0f;

  wait_vmem();
  __syncthreads();

  // one key block: multiply out of `cur`, prefetch the next block into `nxt`
  auto block = [&](int kb, uint8_t *cur, uint8_t *nxt) {
    if (kb + 1 < nkb) att_load<HD>(rk, rv, nxt, head_rows, (int64_t)h * HD, ldv, kb + 1);
    const int valid = (int)min((int64_t)AKV, N - (int64_t)kb * AKV);
    if (valid < AKV) {
      // keys past the end: zero their values so that 0-weight * garbage stays 0
      for (int idx = threadIdx.x; idx < HD * AKV; idx += ATHREADS) {
        const int row = idx / AKV, key = idx % AKV;
        if (key >= valid) {
          const int ps = (int)vt_pos(key);   // physical position of the key in the row
          *reinterpret_cast<uint16_t *>(cur + C::KBYTES + row * C::VROW + (att_slot(ps >> 3, row, 8) << 4) + (ps & 7) * 2) = 0;
        }
      }
      __syncthreads();
    }
    // S^T for 64 keys x 32 queries: two 32-key tiles
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
      s[t] = f32x16{0};
      const int krow = t * 32 + l32;
#pragma unroll
      for (int st = 0; st < KS; st++) {
        const u32x4 kf = *reinterpret_cast<const u32x4 *>(cur + krow * C::KROW + (att_slot(2 * st + hsel, krow, HD / 8) << 4));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qf[st]),
                                                       s[t], 0, 0, 0);
      }
    }
    // online softmax over this block (lane = one query; rows r are keys).  The max is taken
    // on raw scores (the scale c2 > 0 keeps the order); p = 2^(s*c2 - m*c2) with one fma.
    // Keys past the end exist only in the last block.
    if (valid < AKV) {
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int key = t * 32 + 8 * (r / 4) + 4 * hsel + (r % 4);
          if (key >= valid) s[t][r] = -INFINITY;
        }
    }
    float mq[4];
#pragma unroll
    for (int u = 0; u < 4; u++) mq[u] = fmaxf(s[u >> 1][(u & 1) * 8], s[u >> 1][(u & 1) * 8 + 1]);
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        if ((r & 7) > 1) mq[t * 2 + (r >> 3)] = fmaxf(mq[t * 2 + (r >> 3)], s[t][r]);
    float mb = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    m_true = fmaxf(m_true, mb);
    // raise the reference (and rescale what was summed against the old one) only when a
    // lane's scores would exceed it by more than 2^8; the first block always does
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
    const float mc = m_ref * c2;
    float lq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c2, -mc));
        s[t][r] = p;
        lq[t * 2 + (r >> 3)] += p;
      }
    float ls = (lq[0] + lq[1]) + (lq[2] + lq[3]);
    ls += __shfl_xor(ls, 32, 64);
    l_run += ls;
    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int ps = 0; ps < 4; ps++) {
      const int t = ps >> 1, rb = 8 * (ps & 1);
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; j++) pf[j] = (__bf16)s[t][rb + j];
      // keys 16ps+4h..+3 and 16ps+8+4h..+3 sit at positions 16ps+8h..+7: chunk 2ps+h of the row
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        const int row = dt * 32 + l32;
        const u32x4 vf = *reinterpret_cast<const u32x4 *>(cur + C::KBYTES + row * C::VROW + (att_slot(2 * ps + hsel, row, 8) << 4));
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf), pf, acc[dt], 0, 0, 0);
      }
    }
    wait_vmem();
    __syncthreads();
  };
  for (int kb = 0; kb < nkb; kb += 2) {
    block(kb, stage0, stage1);
    if (kb + 1 < nkb) block(kb + 1, stage1, stage0);
  }

  // O[h][q][dim] = O^T / l; lane holds dims dt*32 + 8(r/4) + 4 hsel + r%4 of query qrow
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
