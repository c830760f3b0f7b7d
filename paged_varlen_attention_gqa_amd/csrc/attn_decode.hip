// Decode attention kernel: requests whose packed query rows (S_b * G) fit in
// one 16-column MFMA tile, bf16, head_dim 128, block_size a power of two that
// is a multiple of 16.
//
// A workgroup owns one (request, KV head, split); its NW waves stream
// interleaved 16-key tiles of the split's key range, each wave with its own
// online-softmax state, and merge through LDS at the end. Per tile a wave:
//   * loads K straight into bf16 MFMA A operands (lane: key l%16, 8 dims at
//     32c + 8(l/16)), and V rows as 16-byte pieces (lane: key 4(l/16)+kg,
//     dims 8(l%16)..+7); every load instruction reads whole 64- or 256-byte
//     row segments, and the next tile's loads are in flight during the
//     current tile's arithmetic;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (lane: column l%16, keys
//     4(l/16)+i), scale, relative bias, masks, online softmax;
//   * O += P V with v_mfma_f32_16x16x4_f32: the k slot of MFMA kg is key
//     4(l/16)+kg, which is exactly the S^T element a lane already holds, and
//     output column n of MFMA e is dim 8n+e, which is element e of the V piece
//     the lane loaded. No transpose and no LDS traffic in the key loop.
// All global reads in the key loop are buffer loads from a per-page (or
// per-workgroup) resource, so a lane's address is one 32-bit offset.
//
// Score and bias rule: prhub.com.cn report on vLLM PR #48858, "key source
// snippets" (score_mod_rel_bias); paged-cache layout and the split count:
// docs.vllm.ai inkling_fa4_rel_attention / inkling_fa4_num_splits.
#include "device_common.h"
#include "kernels.h"

namespace relattn {

namespace {

constexpr int kD = 128;
constexpr int kTile = 16;
// A running max is kept until a tile's max exceeds it by this much (log2
// units), so that the accumulator rescale is rare; probabilities stay below
// 2^8 and are accumulated in fp32.
constexpr float kRescaleSlack = 8.0f;

struct TileRegs {
  u32x4_t k[kD / 32];
  u32x4_t v[4];
  uint32_t bias[4];  // raw bf16 bits of the bias for the lane's 4 keys
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_decode_kernel(AttnParams P) {
  __shared__ __attribute__((aligned(16))) float o_lds[NW][16][kD];
  __shared__ float m_lds[NW][16];
  __shared__ float l_lds[NW][16];

  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int split = blockIdx.x;
  int t0, S, L;
  if (!request_bounds(P, b, t0, S, L)) return;
  const int G = P.G;
  const int rows = S * G;
  if (rows > 16) return;  // handled by the general kernel

  const int tid = threadIdx.x;
  // wave index as a scalar, so that the tile loop runs on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;  // column (query row) / K key / V dim group
  const int q = lane >> 4;  // 0..3

  // column n: token n / G of the request, query head g*G + n % G
  const bool col_ok = n < rows;
  const int itok = col_ok ? n / G : 0;
  const int hh = col_ok ? n % G : 0;
  const int h = g * G + hh;
  const int t = t0 + itok;
  const int p = itok + L - S;
  int row_lo = 0, row_hi = 0;
  if (col_ok) visible_range(P, p, L, row_lo, row_hi);

  // key range of the workgroup: union over its first and last token
  int lo_a, hi_a, lo_b, hi_b;
  visible_range(P, L - S, L, lo_a, hi_a);
  visible_range(P, L - 1, L, lo_b, hi_b);
  const int wg_lo = min(lo_a, lo_b);
  const int wg_hi = max(hi_a, hi_b);
  const int kstart = wg_lo & ~(kTile - 1);
  const int c0 = __builtin_amdgcn_readfirstlane(kstart + split * P.dec_chunk);
  const int c1 = min(c0 + P.dec_chunk, wg_hi);
  const int ntiles = __builtin_amdgcn_readfirstlane(c1 > c0 ? (c1 - c0 + kTile - 1) / kTile : 0);

  if (ntiles == 0) {
    // an empty split still tells the combine step it holds nothing
    if (P.splits > 1 && wave == 0 && q == 0 && col_ok)
      P.ws_lse[((int64_t)split * P.T + t) * P.H + h] = kNegInf;
    return;
  }

  // Q^T as the B operand of the QK MFMA
  const int64_t qoff = ((int64_t)t * P.H + h) * kD;
  u32x4_t qreg[kD / 32];
#pragma unroll
  for (int c = 0; c < kD / 32; ++c) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (col_ok) v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(P.q) + qoff + 32 * c + 8 * q);
    qreg[c] = v;
  }

  // lane byte offsets inside a 16-key tile, from the tile's first slot row
  const uint32_t row_bytes = (uint32_t)P.Hkv * kD * 2;  // between consecutive slots
  const uint32_t koff = n * row_bytes + 16u * q;
  uint32_t voff[4];
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) voff[kg] = (4 * q + kg) * row_bytes + 16u * n;

  // relative-bias rows of this workgroup's columns: one resource from the
  // first column's row, lane offsets relative to it
  const int E = P.E;
  const int Em1 = E > 0 ? E - 1 : 0;
  const char* rel_base = E > 0 ? reinterpret_cast<const char*>(P.rel) + ((int64_t)t0 * P.H + g * G) * E * 2
                               : reinterpret_cast<const char*>(P.q);
  const uint32_t rel_lane = E > 0 ? (uint32_t)((itok * P.H + hh) * E) * 2u : 0u;
  const __amdgpu_buffer_rsrc_t rel_rsrc = make_rsrc(rel_base);

  const int bs_log2 = P.bs_log2;
  const int bs_mask = P.bs - 1;
  const int32_t* bt_row = P.block_table + (int64_t)b * P.max_blocks;
  const int npages_req = (L + P.bs - 1) >> bs_log2;

  // page ids of the split, 64 at a time: lane i holds page pbase + i
  int pbase = c0 >> bs_log2;
  auto load_pages = [&](int first) -> int {
    const int idx = first + lane;
    int pg = idx < npages_req ? bt_row[idx] : 0;
    return pg < 0 ? 0 : (pg >= P.num_blocks ? P.num_blocks - 1 : pg);
  };
  int pages = load_pages(pbase);

  const char* kbytes = reinterpret_cast<const char*>(P.k);
  const char* vbytes = reinterpret_cast<const char*>(P.v);
  const int64_t head_bytes = (int64_t)g * kD * 2;

  auto load_tile = [&](TileRegs& R, int j0) {
    const int pidx = j0 >> bs_log2;
    if (pidx - pbase >= 64) {
      pbase = pidx;
      pages = load_pages(pbase);
    }
    const int page = __builtin_amdgcn_readlane(pages, pidx - pbase);
    const int64_t base = (((int64_t)page << bs_log2) + (j0 & bs_mask)) * row_bytes + head_bytes;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbytes + base);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbytes + base);
#pragma unroll
    for (int c = 0; c < kD / 32; ++c)
      R.k[c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(kr, koff + 64u * c, 0, 0));
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
      R.v[kg] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vr, voff[kg], 0, 0));
    // Four consecutive distances, clamped into the row so that the loads are
    // always issued and always in bounds; compute_tile drops the ones
    // outside [0, E). A fixed number of loads per tile keeps the prefetch
    // wait counts exact.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = p - (j0 + 4 * q + i);
      const int dc = d < 0 ? 0 : (d > Em1 ? Em1 : d);
      R.bias[i] = __builtin_amdgcn_raw_buffer_load_b16(rel_rsrc, rel_lane + 2u * dc, 0, 0);
    }
  };

  f32x4_t oacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) oacc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;  // per column (lanes with equal n agree)
  float l_part = 0.f;     // this lane's share of the column's sum

  auto compute_tile = [&](TileRegs& R, int j0) {
    // S^T = K Q^T
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kD / 32; ++c)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, R.k[c]),
                                                  __builtin_bit_cast(bf16x8_t, qreg[c]), s, 0, 0, 0);
    // branch-free, so that every lane consumes its bias registers on every
    // path (a skipped use would leave the loads pending for the wait counter)
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * q + i;
      const uint32_t in_range = (uint32_t)(p - j) < (uint32_t)E ? 0xffffffffu : 0u;
      const float bias = __uint_as_float((R.bias[i] << 16) & in_range);
      const float v = fmaf(s[i], P.scale_log2, bias * kLog2e);
      const bool vis = (j >= row_lo) & (j < row_hi);
      s[i] = vis ? v : kNegInf;
      mx = fmaxf(mx, s[i]);
    }
    mx = wave_max_xor_16_32(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_ref == kNegInf ? 0.f : exp2f(m_ref - m_new);
      m_ref = m_new;
      l_part *= alpha;
      // O rows are columns 4q+i; their alpha lives in lanes 4q+i
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * q + i);
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[e][i] *= a4[i];
    }
    const float m_use = m_ref == kNegInf ? 0.f : m_ref;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = exp2f(s[i] - m_use);
      l_part += s[i];
    }
    // keys past L may hold anything (NaN): their V rows must not reach the MFMA
    if (j0 + kTile > L) {
#pragma unroll
      for (int kg = 0; kg < 4; ++kg)
        if (j0 + 4 * q + kg >= L) R.v[kg] = u32x4_t{0u, 0u, 0u, 0u};
    }
    // O += P V on fp32 MFMA
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const float a = s[kg];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = R.v[kg][e >> 1];
        const float bv = (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
        oacc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, oacc[e], 0, 0, 0);
      }
    }
  };

  // ---- key loop: wave w owns tiles w, w+NW, ...; one tile of loads ahead ----
  // The prefetch is unconditional (the last one re-reads the wave's last
  // tile, from cache) so that the compiler's wait counts stay exact: a
  // conditional load would make it wait for the prefetch as well.
  {
    const int nw = wave < ntiles ? (ntiles - wave + NW - 1) / NW : 0;
    auto j0_of = [&](int i) { return c0 + kTile * (wave + NW * min(i, nw - 1)); };
    TileRegs RA, RB;
    if (nw > 0) {
      load_tile(RA, j0_of(0));
      for (int i = 0; i < nw; i += 2) {
        load_tile(RB, j0_of(i + 1));
        compute_tile(RA, j0_of(i));
        if (i + 1 >= nw) break;
        load_tile(RA, j0_of(i + 2));
        compute_tile(RB, j0_of(i + 1));
      }
    }
  }

  // ---- merge the waves' partial states through LDS ----
  const float l_col = wave_sum_xor_16_32(l_part);
  if (q == 0) {
    m_lds[wave][n] = m_ref;
    l_lds[wave][n] = l_col;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4_t lo4 = {oacc[0][i], oacc[1][i], oacc[2][i], oacc[3][i]};
    f32x4_t hi4 = {oacc[4][i], oacc[5][i], oacc[6][i], oacc[7][i]};
    *reinterpret_cast<f32x4_t*>(&o_lds[wave][4 * q + i][8 * n]) = lo4;
    *reinterpret_cast<f32x4_t*>(&o_lds[wave][4 * q + i][8 * n + 4]) = hi4;
  }
  __syncthreads();

  // thread -> (column c, 8 dims); 16 columns x 16 dim groups
  if (tid >= 256) return;
  const int c = tid >> 4;
  const int dg = tid & 15;
  if (c >= rows) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, m_lds[w][c]);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float Lsum = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = m_lds[w][c];
      if (mw == kNegInf) continue;
      const float sc = exp2f(mw - M);
      Lsum += l_lds[w][c] * sc;
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&o_lds[w][c][8 * dg]);
      const f32x4_t bq = *reinterpret_cast<const f32x4_t*>(&o_lds[w][c][8 * dg + 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(a[e], sc, acc[e]);
        acc[4 + e] = fmaf(bq[e], sc, acc[4 + e]);
      }
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  const int ct = t0 + c / G;
  const int ch = g * G + c % G;
  // acc[e] holds dim 8*dg + e
  if (P.splits == 1) {
    uint16_t* op = reinterpret_cast<uint16_t*>(P.out) + ((int64_t)ct * P.H + ch) * kD + 8 * dg;
    u32x4_t w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                 pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
    *reinterpret_cast<u32x4_t*>(op) = w;
  } else {
    const int64_t slot = ((int64_t)split * P.T + ct) * P.H + ch;
    float* wo = P.ws_o + slot * kD + 8 * dg;
    *reinterpret_cast<f32x4_t*>(wo) = f32x4_t{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4_t*>(wo + 4) = f32x4_t{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    if (dg == 0) P.ws_lse[slot] = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : kNegInf;
  }
}

}  // namespace

bool decode_supported(const AttnParams& P, int dtype_bf16, int head_dim) {
  return dtype_bf16 && head_dim == kD && P.bs_log2 >= 4;
}

int launch_decode(const AttnParams& P, int head_dim, hipStream_t stream) {
  (void)head_dim;
  dim3 grid(P.splits, P.Hkv, P.B);
  if (P.B == 0) return 0;
  if (P.dec_chunk >= 1024)
    hipLaunchKernelGGL((attn_decode_kernel<8>), grid, dim3(512), 0, stream, P);
  else
    hipLaunchKernelGGL((attn_decode_kernel<4>), grid, dim3(256), 0, stream, P);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace relattn
