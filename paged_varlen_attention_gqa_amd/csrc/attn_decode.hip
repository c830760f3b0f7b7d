// Decode attention kernel: requests whose packed query rows (S_b * G) fit in
// one 16-column MFMA tile, bf16, head_dim 128, block_size a power of two that
// is a multiple of 16.
//
// A workgroup owns one (request, KV head, split); its NW waves stream
// interleaved 16-key tiles of the split's key range, each wave with its own
// online-softmax state, and merge through LDS at the end. Each wave has a
// private ring of RING tile slots in LDS that buffer loads fill directly
// (global -> LDS, no registers), RING - 1 tiles ahead of the arithmetic.
// Per tile a wave:
//   * reads K from LDS as bf16 MFMA A operands (lane: key l%16, 8 dims at
//     32c + 8(l/16)) and computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16
//     (lane: column l%16, keys 4(l/16)+i); scale, relative bias, masks and
//     the online softmax stay in that layout;
//   * reads V^T from the row-major V tile with the LDS transpose read
//     (ds_read_b64_tr_b16: lane (g, i) of a 16-lane group g receives
//     V[4g + k][16mb + i], k = 0..3) and accumulates O^T += V^T P^T with
//     v_mfma_f32_16x16x16_bf16, whose B operand is the S^T layout itself.
// The 16-byte chunks of every LDS row are XOR-swizzled by a function of the
// row so that both read patterns are free of bank conflicts.
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
constexpr int kRowBytes = kD * 2;              // one key row of K or V in LDS
constexpr int kHalfSlot = kTile * kRowBytes;   // K (or V) part of a slot: 4 KB
constexpr int kSlotBytes = 2 * kHalfSlot;      // one tile: K then V, 8 KB
// A running max is kept until a tile's max exceeds it by this much (log2
// units), so that the accumulator rescale is rare; probabilities stay below
// 2^8.
constexpr float kRescaleSlack = 8.0f;

// waves per workgroup and ring depth (tiles per wave in LDS)
#ifndef REL_ATTN_DECODE_WAVES
#define REL_ATTN_DECODE_WAVES 4
#endif
#ifndef REL_ATTN_DECODE_RING
#define REL_ATTN_DECODE_RING 2
#endif
#ifndef REL_ATTN_DECODE_HEADS_FIRST
#define REL_ATTN_DECODE_HEADS_FIRST 1
#endif
constexpr int kDecodeWaves = REL_ATTN_DECODE_WAVES;
constexpr int kDecodeRing = REL_ATTN_DECODE_RING;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// Chunk swizzle of LDS row r (16 chunks of 16 bytes per row): a bijection of
// 0..15 that maps rows 4g..4g+3 to four distinct even values (transpose
// reads) and all 16 rows to distinct values (K operand reads).
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// global -> LDS copy of 1 KB per instruction: lane l writes bytes
// [16l, 16l+16) of the destination block.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}

template <int NW, int RING>
__global__ __launch_bounds__(NW * 64) void attn_decode_kernel(AttnParams P) {
  // One LDS object per ring slot, so that the compiler waits for exactly the
  // copies a read depends on; wave w owns bytes [w*8K, (w+1)*8K) of each.
  __shared__ __attribute__((aligned(1024))) char ring0[NW * kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[NW * kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[RING > 2 ? NW * kSlotBytes : 16];
  __shared__ float m_lds[NW][16];
  __shared__ float l_lds[NW][16];
  static_assert(RING == 2 || RING == 3, "ring depth");

#if REL_ATTN_DECODE_HEADS_FIRST
  // the KV heads of one (request, split) are neighbours in launch order, so
  // they walk the same pages at about the same time (DRAM row locality: the
  // heads of one slot share a cache row)
  const int b = blockIdx.z;
  const int g = blockIdx.x;
  const int split = blockIdx.y;
#else
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int split = blockIdx.x;
#endif
  int t0, S, L;
  if (!request_bounds(P, b, t0, S, L)) return;
  const int G = P.G;
  const int rows = S * G;
  if (rows > 16) return;  // handled by the general kernel

  const int tid = threadIdx.x;
  // wave index as a scalar, so that the tile loop runs on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;  // column (query row) / K row / transpose-read lane
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
    // No visible key: the row's output is zero, and an empty split still
    // tells the combine step that it holds nothing. Lane (n, q) of wave 0
    // writes dims 32q .. 32q+31 of column n.
    if (wave == 0 && col_ok) {
      if (P.splits == 1) {
        uint16_t* op = reinterpret_cast<uint16_t*>(P.out) + ((int64_t)t * P.H + h) * kD + 32 * q;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(op + 8 * i) = u32x4_t{0u, 0u, 0u, 0u};
      } else {
        const int64_t slot = ((int64_t)split * P.T + t) * P.H + h;
        float* wo = P.ws_o + slot * kD + 32 * q;
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4_t*>(wo + 4 * i) = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (q == 0) P.ws_lse[slot] = kNegInf;
      }
    }
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

  // copy offsets: copy instruction r of a tile fills LDS rows 4r..4r+3; lane
  // l lands in row 4r + l/16 at chunk position l%16, which holds logical
  // chunk (l%16) ^ swz(row) of that key's row
  const uint32_t row_bytes = (uint32_t)P.Hkv * kD * 2;  // between consecutive slots in the cache
  uint32_t cp_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * r + q;
    cp_off[r] = (uint32_t)row * row_bytes + 16u * (uint32_t)(n ^ swz(row));
  }
  // K operand reads: row n, logical chunk 4c + q
  uint32_t k_rd[kD / 32];
#pragma unroll
  for (int c = 0; c < kD / 32; ++c) k_rd[c] = (uint32_t)(n * kRowBytes + 16 * ((4 * c + q) ^ swz(n)));
  // transpose reads of V: lane (q, n) points at row 4q + n/4, 8 bytes at
  // dims 16mb + 4(n%4), i.e. logical chunk 2mb + (n%4)/2, half n%2
  uint32_t v_rd[kD / 16];
  {
    const int row = 4 * q + (n >> 2);
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb)
      v_rd[mb] = (uint32_t)(kHalfSlot + row * kRowBytes + 16 * ((2 * mb + ((n & 3) >> 1)) ^ swz(row)) + 8 * (n & 1));
  }

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
  char* const my0 = ring0 + wave * kSlotBytes;
  char* const my1 = ring1 + wave * kSlotBytes;
  char* const my2 = ring2 + (RING > 2 ? wave * kSlotBytes : 0);

  // keys that can carry a bias for some column: (p_min - E, p_max]
  const int band_lo = __builtin_amdgcn_readfirstlane((L - S) - E + 1);
  const int band_hi = __builtin_amdgcn_readfirstlane(L - 1);

  // start the copy of the tile at key j0 into a slot; its bias goes to bias[]
  auto issue = [&](char* slot, uint32_t (&bias)[4], int j0) {
    // Bias first: the copies issued after it are then the only loads a later
    // wait has to leave in flight, whether or not this tile loaded a bias.
    // Four consecutive distances, clamped into the row (always in bounds);
    // the arithmetic drops the ones outside [0, E).
    if (E > 0 && j0 + kTile > band_lo && j0 <= band_hi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = p - (j0 + 4 * q + i);
        const int dc = d < 0 ? 0 : (d > Em1 ? Em1 : d);
        bias[i] = __builtin_amdgcn_raw_buffer_load_b16(rel_rsrc, rel_lane + 2u * dc, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[i] = 0u;
    }
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
    for (int r = 0; r < 4; ++r) dma16(kr, slot + 1024 * r, cp_off[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) dma16(vr, slot + kHalfSlot + 1024 * r, cp_off[r]);
    // the copies wrote LDS behind the compiler's back
    asm volatile("" ::: "memory");
  };

  f32x4_t oacc[kD / 16];  // O^T: lane (q, n) holds dims 16mb + 4q + i of column n
#pragma unroll
  for (int mb = 0; mb < kD / 16; ++mb) oacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;  // per column (lanes with equal n agree)
  float l_part = 0.f;     // this lane's share of the column's sum

  auto compute = [&](const char* slot, const uint32_t (&bias)[4], int j0) {
    // S^T = K Q^T
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kD / 32; ++c) {
      const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(slot + k_rd[c]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf),
                                                  __builtin_bit_cast(bf16x8_t, qreg[c]), s, 0, 0, 0);
    }
    // branch-free, so that every lane consumes its bias registers on every
    // path (a skipped use would leave the loads pending for the wait counter)
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * q + i;
      const uint32_t in_range = (uint32_t)(p - j) < (uint32_t)E ? 0xffffffffu : 0u;
      const float bv = __uint_as_float((bias[i] << 16) & in_range);
      const float v = fmaf(s[i], P.scale_log2, bv * kLog2e);
      const bool vis = (j >= row_lo) & (j < row_hi);
      s[i] = vis ? v : kNegInf;
      mx = fmaxf(mx, s[i]);
    }
    mx = wave_max_xor_16_32(mx);
    // The reference max only moves when a tile's max exceeds it by the slack
    // (probabilities then stay below 2^8). The rescale is applied on every
    // tile, branch-free; alpha is 1 unless the reference moved.
    const float m_new = mx > m_ref + kRescaleSlack ? mx : m_ref;
    const float alpha = m_ref == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
    m_ref = m_new;
    l_part *= alpha;
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb) oacc[mb] *= alpha;
    const float m_use = m_ref == kNegInf ? 0.f : m_ref;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
      l_part += s[i];
    }
    const u32x2_t pb = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
    // keys past L may hold anything (NaN) and 0 * NaN is NaN: mask their V
    // elements (this lane's transposed operand holds keys 4q..4q+3)
    const bool tail = j0 + kTile > L;
    u32x2_t vmask = {0xffffffffu, 0xffffffffu};
    if (tail) {
      const int k0 = j0 + 4 * q;
      vmask[0] = (k0 < L ? 0xffffu : 0u) | (k0 + 1 < L ? 0xffff0000u : 0u);
      vmask[1] = (k0 + 2 < L ? 0xffffu : 0u) | (k0 + 3 < L ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb) {
      v4i16_t vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16_t*)(slot + v_rd[mb]));
      if (tail) vf = __builtin_bit_cast(v4i16_t, __builtin_bit_cast(u32x2_t, vf) & vmask);
      oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, __builtin_bit_cast(i16x4_t, pb), oacc[mb], 0, 0, 0);
    }
  };

  // ---- key loop: wave w owns tiles w, w+NW, ...; RING-1 tiles in flight ----
  // Inside the loop every step issues one tile's copies unconditionally, so
  // the compiler's wait counts stay exact (a conditional load would make it
  // wait for the prefetch too); the last RING-1 tiles are computed after it.
  {
    const int nw = wave < ntiles ? (ntiles - wave + NW - 1) / NW : 0;
    auto j0_of = [&](int i) { return c0 + kTile * (wave + NW * i); };
    uint32_t b0[4], b1[4], b2[4];
    if constexpr (RING == 3) {
      if (nw > 0) issue(my0, b0, j0_of(0));
      if (nw > 1) issue(my1, b1, j0_of(1));
      int i = 0;
      for (; i + 2 < nw; i += 3) {
        issue(my2, b2, j0_of(i + 2));
        compute(my0, b0, j0_of(i));
        if (i + 3 >= nw) { compute(my1, b1, j0_of(i + 1)); compute(my2, b2, j0_of(i + 2)); i = nw; break; }
        issue(my0, b0, j0_of(i + 3));
        compute(my1, b1, j0_of(i + 1));
        if (i + 4 >= nw) { compute(my2, b2, j0_of(i + 2)); compute(my0, b0, j0_of(i + 3)); i = nw; break; }
        issue(my1, b1, j0_of(i + 4));
        compute(my2, b2, j0_of(i + 2));
      }
      // 0..2 tiles left, in slots i%3 and (i+1)%3 (i is a multiple of 3 here)
      if (i < nw) compute(my0, b0, j0_of(i));
      if (i + 1 < nw) compute(my1, b1, j0_of(i + 1));
    } else {
      if (nw > 0) issue(my0, b0, j0_of(0));
      int i = 0;
      for (; i + 1 < nw; i += 2) {
        issue(my1, b1, j0_of(i + 1));
        compute(my0, b0, j0_of(i));
        if (i + 2 >= nw) { compute(my1, b1, j0_of(i + 1)); i = nw; break; }
        issue(my0, b0, j0_of(i + 2));
        compute(my1, b1, j0_of(i + 1));
      }
      if (i < nw) compute(my0, b0, j0_of(i));
    }
    (void)b2;
  }

  // ---- merge the waves' partial states through LDS (slot 0 of each wave) ----
  const float l_col = wave_sum_xor_16_32(l_part);
  if (q == 0) {
    m_lds[wave][n] = m_ref;
    l_lds[wave][n] = l_col;
  }
  float* const o_my = reinterpret_cast<float*>(my0);  // [16 columns][kD] fp32
#pragma unroll
  for (int mb = 0; mb < kD / 16; ++mb)
    *reinterpret_cast<f32x4_t*>(&o_my[n * kD + 16 * mb + 4 * q]) = oacc[mb];
  __syncthreads();

  // thread -> (column c, 8 dims); 16 columns x 16 dim groups
  for (int item = tid; item < 256; item += NW * 64) {
    const int c = item >> 4;
    const int dg = item & 15;
    if (c >= rows) break;
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
        const float* ow = reinterpret_cast<const float*>(ring0 + w * kSlotBytes) + c * kD + 8 * dg;
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(ow);
        const f32x4_t bq = *reinterpret_cast<const f32x4_t*>(ow + 4);
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
}

}  // namespace

bool decode_supported(const AttnParams& P, int dtype_bf16, int head_dim) {
  return dtype_bf16 && head_dim == kD && P.bs_log2 >= 4;
}

int launch_decode(const AttnParams& P, int head_dim, hipStream_t stream) {
  (void)head_dim;
#if REL_ATTN_DECODE_HEADS_FIRST
  dim3 grid(P.Hkv, P.splits, P.B);
#else
  dim3 grid(P.splits, P.Hkv, P.B);
#endif
  if (P.B == 0) return 0;
  hipLaunchKernelGGL((attn_decode_kernel<kDecodeWaves, kDecodeRing>), grid, dim3(kDecodeWaves * 64), 0, stream, P);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace relattn
