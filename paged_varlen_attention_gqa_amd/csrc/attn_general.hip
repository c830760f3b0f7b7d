// General attention kernel: any query length, bf16 or fp32, head_dim 64/128.
//
// One workgroup (4 waves) owns 64 packed query rows of one (request, KV head):
// row r of a request is token r / G, query head kv_head * G + r % G, so the G
// query heads that share a KV head (grouped-query attention) share every K/V
// tile. The workgroup walks its share of the key range in 64-key tiles that
// are gathered through the block table into LDS (K row-major, V transposed
// for bf16). Each wave owns 16 rows and computes S^T = K Q^T with MFMA,
// adds the relative bias, masks, updates an online softmax in the log2
// domain, and accumulates O^T += V^T P^T with MFMA.
//
// Score and bias rule: prhub.com.cn report on vLLM PR #48858, "key source
// snippets" (score_mod_rel_bias); tensor layouts: docs.vllm.ai
// inkling_fa4_rel_attention.
#include "device_common.h"
#include "kernels.h"

namespace relattn {

namespace {

constexpr int kRows = 64;   // query rows per workgroup
constexpr int kKeys = 64;   // keys per LDS tile

template <bool BF16, int D>
struct GeneralCfg {
  using elem_t = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int kKPad = BF16 ? 8 : 4;          // K row padding (elements)
  static constexpr int kKStride = D + kKPad;
  // bf16: V^T [D][kKeys + pad];  fp32: V [kKeys][D + pad]
  static constexpr int kVStride = BF16 ? (kKeys + 8) : (D + 4);
  static constexpr int kVRows = BF16 ? D : kKeys;
  static constexpr int kQRegs = BF16 ? D / 32 : D / 4;  // B-operand registers for Q
};

template <bool BF16, int D>
__global__ __launch_bounds__(256) void attn_general_kernel(AttnParams P) {
  using Cfg = GeneralCfg<BF16, D>;
  using elem_t = typename Cfg::elem_t;
  __shared__ __attribute__((aligned(16))) elem_t k_lds[kKeys * Cfg::kKStride];
  __shared__ __attribute__((aligned(16))) elem_t v_lds[Cfg::kVRows * Cfg::kVStride];

  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int qt = blockIdx.x / P.splits;
  const int split = blockIdx.x % P.splits;
  int t0, S, L;
  if (!request_bounds(P, b, t0, S, L)) return;
  const int G = P.G;
  const int nrows = S * G;
  if (P.mode == 1 && nrows <= 16) return;
  const int r0 = qt * kRows;
  if (r0 >= nrows) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 15;   // row within the wave's 16-row tile / MFMA column
  const int lq = lane >> 4;   // 0..3

  // this lane's query row
  const int r = r0 + wave * 16 + lr;
  const bool row_ok = r < nrows;
  const int itok = row_ok ? r / G : 0;
  const int h = g * G + (row_ok ? r % G : 0);
  const int t = t0 + itok;
  const int p = itok + L - S;
  int row_lo = 0, row_hi = 0;
  if (row_ok) visible_range(P, p, L, row_lo, row_hi);

  // key range of the whole workgroup (union of its rows)
  const int ia = r0 / G;
  const int ib = (min(r0 + kRows, nrows) - 1) / G;
  int lo_a, hi_a, lo_b, hi_b;
  visible_range(P, ia + L - S, L, lo_a, hi_a);
  visible_range(P, ib + L - S, L, lo_b, hi_b);
  const int wg_lo = min(lo_a, lo_b);
  const int wg_hi = max(hi_a, hi_b);
  const int kstart = wg_lo & ~(kKeys - 1);
  const int ntiles = wg_hi > wg_lo ? (wg_hi - kstart + kKeys - 1) / kKeys : 0;
  const int tps = (ntiles + P.splits - 1) / P.splits;
  const int tile_begin = split * tps;
  const int tile_end = min(ntiles, tile_begin + tps);

  const elem_t* qp = reinterpret_cast<const elem_t*>(P.q);
  const elem_t* kp = reinterpret_cast<const elem_t*>(P.k);
  const elem_t* vp = reinterpret_cast<const elem_t*>(P.v);
  const elem_t* relp = reinterpret_cast<const elem_t*>(P.rel);
  const int64_t rel_row = ((int64_t)t * P.H + h) * P.E;

  // Q as the MFMA B operand (columns = rows of this wave)
  u32x4_t qreg_bf[BF16 ? Cfg::kQRegs : 1];
  float qreg_f[BF16 ? 1 : Cfg::kQRegs];
  const int64_t qoff = ((int64_t)t * P.H + h) * D;
  if constexpr (BF16) {
#pragma unroll
    for (int c = 0; c < Cfg::kQRegs; ++c) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4_t*>(qp + qoff + 32 * c + 8 * lq);
      qreg_bf[c] = v;
    }
  } else {
#pragma unroll
    for (int c = 0; c < Cfg::kQRegs; ++c) qreg_f[c] = row_ok ? qp[qoff + 4 * c + lq] : 0.f;
  }

  f32x4_t o_acc[D / 16];
#pragma unroll
  for (int m = 0; m < D / 16; ++m) o_acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;
  float l_run = 0.f;   // lane-partial row sum

  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int j0 = kstart + tile * kKeys;
    __syncthreads();
    // ---- gather the K/V tile through the block table into LDS ----
    if constexpr (BF16) {
      constexpr int kChunks = D / 8;  // 16-byte chunks per row
      for (int c = tid; c < kKeys * kChunks; c += 256) {
        const int key = c / kChunks, dc = c % kChunks;
        const int j = j0 + key;
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (j < L) val = *reinterpret_cast<const u32x4_t*>(kp + kv_row(P, b, g, j) * D + 8 * dc);
        *reinterpret_cast<u32x4_t*>(&k_lds[key * Cfg::kKStride + 8 * dc]) = val;
      }
      // V transposed: each item is 4 keys x 8 dims
      for (int it = tid; it < (kKeys / 4) * kChunks; it += 256) {
        const int kg = it / kChunks, dc = it % kChunks;
        u32x4_t vv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + 4 * kg + e;
          vv[e] = u32x4_t{0u, 0u, 0u, 0u};
          if (j < L) vv[e] = *reinterpret_cast<const u32x4_t*>(vp + kv_row(P, b, g, j) * D + 8 * dc);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // dims 8dc+2w (low halves) and 8dc+2w+1 (high halves)
          u32x2_t lo2 = {(vv[0][w] & 0xffffu) | (vv[1][w] << 16), (vv[2][w] & 0xffffu) | (vv[3][w] << 16)};
          u32x2_t hi2 = {(vv[0][w] >> 16) | (vv[1][w] & 0xffff0000u),
                         (vv[2][w] >> 16) | (vv[3][w] & 0xffff0000u)};
          *reinterpret_cast<u32x2_t*>(&v_lds[(8 * dc + 2 * w) * Cfg::kVStride + 4 * kg]) = lo2;
          *reinterpret_cast<u32x2_t*>(&v_lds[(8 * dc + 2 * w + 1) * Cfg::kVStride + 4 * kg]) = hi2;
        }
      }
    } else {
      constexpr int kChunks = D / 4;
      for (int c = tid; c < kKeys * kChunks; c += 256) {
        const int key = c / kChunks, dc = c % kChunks;
        const int j = j0 + key;
        f32x4_t kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
        if (j < L) {
          const int64_t off = kv_row(P, b, g, j) * D + 4 * dc;
          kv = *reinterpret_cast<const f32x4_t*>(kp + off);
          vv = *reinterpret_cast<const f32x4_t*>(vp + off);
        }
        *reinterpret_cast<f32x4_t*>(&k_lds[key * Cfg::kKStride + 4 * dc]) = kv;
        *reinterpret_cast<f32x4_t*>(&v_lds[key * Cfg::kVStride + 4 * dc]) = vv;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for the four 16-key sub-tiles ----
    f32x4_t s[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
#pragma unroll
        for (int c = 0; c < Cfg::kQRegs; ++c) {
          u32x4_t a = *reinterpret_cast<const u32x4_t*>(&k_lds[(16 * st + lr) * Cfg::kKStride + 32 * c + 8 * lq]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, qreg_bf[c]), acc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < Cfg::kQRegs; ++c) {
          float a = k_lds[(16 * st + lr) * Cfg::kKStride + 4 * c + lq];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qreg_f[c], acc, 0, 0, 0);
        }
      }
      s[st] = acc;
    }

    // ---- scale, relative bias, mask (log2 domain) ----
    float mx = kNegInf;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 16 * st + 4 * lq + e;
        const bool vis = (j >= row_lo) && (j < row_hi);
        float bias = 0.f;
        const int d = p - j;
        if (vis && d >= 0 && d < P.E) {
          if constexpr (BF16) bias = bf16_bits_to_f32(relp[rel_row + d]);
          else bias = relp[rel_row + d];
        }
        const float v = vis ? fmaf(s[st][e], P.scale_log2, bias * kLog2e) : kNegInf;
        s[st][e] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = wave_max_xor_16_32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = exp2f(s[st][e] - m_use);
        s[st][e] = pv;
        psum += pv;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) o_acc[m] *= alpha;

    // ---- O^T += V^T P^T ----
    if constexpr (BF16) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        u32x2_t pb = {pack_bf16x2(s[st][0], s[st][1]), pack_bf16x2(s[st][2], s[st][3])};
#pragma unroll
        for (int m = 0; m < D / 16; ++m) {
          u32x2_t a = *reinterpret_cast<const u32x2_t*>(&v_lds[(16 * m + lr) * Cfg::kVStride + 16 * st + 4 * lq]);
          o_acc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                               __builtin_bit_cast(i16x4_t, pb), o_acc[m], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int m = 0; m < D / 16; ++m) {
            float a = v_lds[(16 * st + 4 * lq + e) * Cfg::kVStride + 16 * m + lr];
            o_acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s[st][e], o_acc[m], 0, 0, 0);
          }
    }
  }

  // ---- epilogue ----
  const float l_tot = wave_sum_xor_16_32(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (P.splits == 1) {
    elem_t* op = reinterpret_cast<elem_t*>(P.out) + qoff;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      const int d = 16 * m + 4 * lq;
      if constexpr (BF16) {
        u32x2_t w = {pack_bf16x2(o_acc[m][0] * inv, o_acc[m][1] * inv),
                     pack_bf16x2(o_acc[m][2] * inv, o_acc[m][3] * inv)};
        *reinterpret_cast<u32x2_t*>(op + d) = w;
      } else {
        *reinterpret_cast<f32x4_t*>(op + d) = o_acc[m] * inv;
      }
    }
  } else {
    const int64_t slot = ((int64_t)split * P.T + t) * P.H + h;
    float* wo = P.ws_o + slot * D;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) *reinterpret_cast<f32x4_t*>(wo + 16 * m + 4 * lq) = o_acc[m] * inv;
    if (lq == 0) P.ws_lse[slot] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

int launch_general(const AttnParams& P, int dtype_bf16, int head_dim, hipStream_t stream) {
  const int qtiles = (P.max_q * P.G + kRows - 1) / kRows;
  dim3 grid(qtiles * P.splits, P.Hkv, P.B);
  dim3 block(256);
  if (grid.x == 0 || P.B == 0) return 0;
  if (dtype_bf16) {
    if (head_dim == 128) hipLaunchKernelGGL((attn_general_kernel<true, 128>), grid, block, 0, stream, P);
    else hipLaunchKernelGGL((attn_general_kernel<true, 64>), grid, block, 0, stream, P);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((attn_general_kernel<false, 128>), grid, block, 0, stream, P);
    else hipLaunchKernelGGL((attn_general_kernel<false, 64>), grid, block, 0, stream, P);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace relattn
