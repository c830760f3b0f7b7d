// Prefill attention kernel: requests with more than 16 packed query rows,
// bf16, head_dim 128, block_size a power of two that is a multiple of 16.
//
// A workgroup (8 waves) owns 256 packed rows of one (request, KV head): row
// r is token r / G and query head kv_head * G + r % G, so the G query heads
// that share a KV head share every K/V tile. Wave w owns rows 32w..32w+31
// as the 32 columns of S^T = K Q^T. Per 64-key tile (two 32-key sub-tiles):
//   * buffer-to-LDS copies bring the K/V tile (shared by the workgroup, one
//     tile ahead) and each wave's slice of relative bias (two tiles ahead)
//     into rings in LDS; a K/V copy names its page by a scalar offset into
//     one resource per cache;
//   * K rows are stored permuted inside each sub-tile: LDS row
//     m = 8i + 4h + k holds key 16h + 4i + k, so that output register a of
//     lane (h, n) of v_mfma_f32_32x32x16_bf16 is key 16h + a;
//   * the relative bias is added by the matrix cores too: two more MFMAs per
//     sub-tile multiply a constant one-hot selection matrix by the bias as
//     the B operand, whose 8 k slots per lane are 8 consecutive entries of
//     one rel_logits row (16-byte pieces of one 128-byte run per row and
//     tile, copied into aligned LDS slots). They start the sub-tile's score accumulator, and
//     the QK^T MFMAs accumulate on top. The selection value is
//     1/softmax_scale when that is a bf16 number; otherwise it is 1 and the
//     accumulator is multiplied by 1/softmax_scale in fp32 before the QK^T
//     MFMAs. Either way the softmax sees softmax_scale * (q.k + bias /
//     softmax_scale) with the bias exact to fp32 rounding;
//   * V^T operands come from the row-major V tile through the LDS transpose
//     read (lane (g, i) of a 16-lane group receives V[4g + k][col0 + i]);
//     O^T += V^T P^T takes the probabilities, packed to bf16, as its B
//     operand;
//   * softmax in the S^T layout: each query column lives in two lanes
//     (l and l ^ 32), so a row max or sum is one lane swap.
// Chunks of every K/V row in LDS are XOR-swizzled so that the K operand
// reads and the transpose reads are free of bank conflicts.
//
// Score and bias rule: prhub.com.cn report on vLLM PR #48858, "key source
// snippets" (score_mod_rel_bias); tensor layouts: docs.vllm.ai
// inkling_fa4_rel_attention.
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

namespace relattn {

namespace {

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kRowsWG = 32 * kWaves;  // packed query rows per workgroup
constexpr int kKeys = 64;             // keys per tile (one stage of the key loop)
constexpr int kSub = 32;              // keys per MFMA sub-tile
constexpr int kRowBytes = kD * 2;
constexpr int kSubBytes = kSub * kRowBytes;  // K (or V) rows of a sub-tile: 8 KB
constexpr int kHalf = kKeys * kRowBytes;     // K (or V) part of a tile: 16 KB
constexpr int kKV = 2 * kHalf;               // 32 KB
constexpr int kBiasWave = 32 * kKeys * 2;    // one wave's bias slice of a tile: 4 KB
constexpr int kKvSlots = 2;                  // K/V ring: copies 1 tile ahead
constexpr int kBiasSlots = 3;                // bias ring: copies 2 tiles ahead
constexpr float kRescaleSlack = 8.0f;     // log2 units, as in the decode kernel

typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Buffer resource (base, size in bytes; out-of-range reads return 0) as the
// four scalar words of the descriptor.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}


// a buffer offset past every resource's range (resources here span less
// than 2 GB): such a copy returns zeros without a memory access
constexpr uint32_t kOutOfRange = 0x80000000u;

// chunk swizzle of K LDS row r: a bijection of 0..15, so that the 16 rows
// of a K operand read (16 lanes of 16 bytes each) fall on distinct chunks
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// chunk swizzle of V LDS row r: 4 (r % 4), so that the four consecutive rows
// of a transpose read land on different chunk groups
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 2; }

// global -> LDS copy of 1 KB per instruction: lane l writes bytes
// [16l, 16l+16) of the LDS block at lds. Issued from inline assembly so that
// the compiler does not guard the LDS reads with waits of its own: it cannot
// tell which LDS bytes such a copy writes, and its conservative waits (for
// copies into other buffers) would stall the prefetch. Every read of copied
// data is preceded by an explicit wait_vm<N> and a barrier instead (both
// fenced against compiler reordering), and a copy only writes a slot that
// no wave reads until then, so the statement needs no memory clobber. It
// sets M0 (the copy's LDS base) itself; nothing else in this kernel keeps a
// value in M0.
__device__ __forceinline__ void dma16(const u32x4_t rsrc, char* lds, uint32_t voff) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v), "v"(voff), "s"(rsrc)
               : "m0");
#pragma clang diagnostic pop
}

// the same copy with a scalar byte offset added to every lane's offset
__device__ __forceinline__ void dma16_soff(const u32x4_t rsrc, char* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
               : "m0");
#pragma clang diagnostic pop
}

// workgroup execution barrier without a memory fence; the empty asm keeps the
// compiler from moving memory operations across it
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Entry x (16 bits each, x = 0..7) of the result is entry x + s of v, zero
// where x + s falls outside 0..7.
__device__ __forceinline__ u32x4_t shift_entries(u32x4_t v, int s) {
  unsigned __int128 w = (unsigned __int128)v[0] | ((unsigned __int128)v[1] << 32) |
                        ((unsigned __int128)v[2] << 64) | ((unsigned __int128)v[3] << 96);
  if (s >= 8 || s <= -8)
    w = 0;
  else if (s >= 0)
    w >>= 16 * s;
  else
    w <<= -16 * s;
  return u32x4_t{(uint32_t)w, (uint32_t)(w >> 32), (uint32_t)(w >> 64), (uint32_t)(w >> 96)};
}

// c + the two bf16 halves of w (v_dot2_f32_bf16 against (1, 1))
__device__ __forceinline__ float dot2_bf16_ones(uint32_t w, float c) {
  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  const bf16x2v_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w), one, c, false);
}

// the middle value of x, 0 and hi (x clamped into [0, hi] for hi >= 0)
__device__ __forceinline__ uint32_t clamp0(int x, int hi) {
  uint32_t r;
  asm("v_med3_i32 %0, %1, 0, %2" : "=v"(r) : "v"(x), "s"(__builtin_amdgcn_readfirstlane(hi)));
  return r;
}

__device__ __forceinline__ float lane_swap32_max(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float lane_swap32_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// block_table is passed again as a restrict-qualified argument so that page
// lookups compile to scalar loads (a vector load would make the next wait for
// it also wait for the copies in flight)
// kWide: a cache spans 4 GB or more, so that K/V copies build a resource
// per page instead of passing a 32-bit offset
// kExactSel: 1/softmax_scale (inv_scale) is a bf16 number and selects the
// bias directly
template <bool kWide, bool kExactSel>
__global__ __launch_bounds__(kWaves * 64) void attn_prefill_kernel(AttnParams P,
                                                                 const int32_t* __restrict__ block_table,
                                                                 float inv_scale) {
  // the K/V ring, then the bias ring (160 KB)
  __shared__ __attribute__((aligned(1024))) char lds[kKvSlots * kKV + kBiasSlots * kWaves * kBiasWave];
  char* const kv_buf = lds;
  char* const bias_buf = lds + kKvSlots * kKV;

  // Dispatch order (the linear workgroup id): KV head fastest, then query
  // tile (longest causal key range first), then request. Workgroups go to
  // the 8 XCDs in turn, so that with 8 KV heads each XCD works through one
  // head of one request at a time and its L2 serves that K/V stream to all
  // of them (measured: faster than tile-fastest or request-fastest orders).
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int g = lin % gridDim.y;
  const int bx = (lin / gridDim.y) % gridDim.x;
  const int b = lin / (gridDim.y * gridDim.x);
  const int qtiles = gridDim.x / P.splits;
  const int qt = qtiles - 1 - bx / P.splits;
  const int split = bx % P.splits;
  int t0, S, L;
  if (!request_bounds(P, b, t0, S, L)) return;
  const int G = P.G;
  const int nrows = S * G;
  if (nrows <= 16) return;  // the decode kernel handles these
  const int r0 = qt * kRowsWG;
  if (r0 >= nrows) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;  // query column of this lane (within the wave)
  const int h = lane >> 5;  // which 16 keys of a 32-key half this lane holds

  const int r = r0 + 32 * wave + n;
  const bool row_ok = r < nrows;
  const int itok = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const int t = t0 + itok;
  const int p = itok + L - S;
  int row_lo = 0, row_hi = 0;
  if (row_ok) visible_range(P, p, L, row_lo, row_hi);

  // key range of the workgroup (union of its rows)
  const int ia = r0 / G;
  const int ib = (min(r0 + kRowsWG, nrows) - 1) / G;
  int lo_a, hi_a, lo_b, hi_b;
  visible_range(P, ia + L - S, L, lo_a, hi_a);
  visible_range(P, ib + L - S, L, lo_b, hi_b);
  const int wg_lo = min(lo_a, lo_b);
  const int wg_hi = max(hi_a, hi_b);
  const int lo_max = max(lo_a, lo_b);  // every row sees [lo_max, hi_min)
  const int hi_min = min(hi_a, hi_b);
  const int kstart = wg_lo & ~(kKeys - 1);
  const int ntiles = wg_hi > wg_lo ? (wg_hi - kstart + kKeys - 1) / kKeys : 0;
  const int tps = (ntiles + P.splits - 1) / P.splits;
  const int tile_begin = __builtin_amdgcn_readfirstlane(split * tps);
  const int tile_end = __builtin_amdgcn_readfirstlane(min(ntiles, tile_begin + tps));

  // Q^T as the B operand: lane (h, n) holds dims 16kk + 8h .. +7 of its row
  u32x4_t qreg[kD / 16];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(P.q) + ((int64_t)t * P.H + hq) * kD;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4_t*>(qp + 16 * kk + 8 * h);
      qreg[kk] = v;
    }
    // wait for q here, once: the compiler does not count the copies issued
    // in the key loop, so a first use of q inside the loop would come with a
    // wait for every copy in flight
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) asm volatile("" ::"v"(qreg[kk]));
  }

  // ---- K/V copy geometry ----
  // wave w copies keys 4w..4w+3 of each sub-tile (inside one page segment) with
  // one instruction for K and one for V; lane l copies one 16-byte chunk of
  // key 4w + l/16. K key 16h' + 4i + kk goes to LDS row 8i + 4h' + kk, so
  // that output register a of lane (h, n) of the QK MFMA is key 16h + a.
  const uint32_t row_bytes = (uint32_t)P.Hkv * kD * 2;
  uint32_t k_src, v_src;
  int k_dst, v_dst;
  {
    const int key = 4 * wave;  // first key of the wave's copy (tile-relative)
    const int krow0 = 8 * ((key & 15) >> 2) + 4 * (key >> 4);
    const int krow = krow0 + (lane >> 4);
    const int vrow = key + (lane >> 4);
    k_src = (uint32_t)(lane >> 4) * row_bytes + 16u * (uint32_t)((lane & 15) ^ swz(krow));
    v_src = (uint32_t)(lane >> 4) * row_bytes + 16u * (uint32_t)((lane & 15) ^ swz_v(vrow));
    k_dst = krow0 * kRowBytes;          // + kSubBytes * sub-tile
    v_dst = kHalf + key * kRowBytes;    // + kSubBytes * sub-tile
  }
  // K operand read of step kk: row n, logical chunk 2kk + h; the
  // chunk is (2kk) ^ (h ^ swz(n)) as 2kk and h occupy disjoint bits
  uint32_t k_rd[kD / 16];
#pragma unroll
  for (int kk = 0; kk < kD / 16; ++kk)
    k_rd[kk] = (uint32_t)(n * kRowBytes + 16 * ((2 * kk) ^ (h ^ swz(n & 15))));
  // transpose reads of V for (block kb, dim tile mt, group sr): lane
  // (h, n), j = n%16, points at row 16h + 8kb + 4sr + j/4, logical chunk
  // 4mt + 2(n/16) + (j%4)/2 (elements 32mt + 16(n/16) + 4(j%4) ..), half
  // j%2. The 32 lanes of a read cover 4 rows x 64 bytes; with the V swizzle
  // 4 (row % 4) the four rows fall on different chunk groups, so the read
  // touches every bank twice (no conflicts), and the chunk is
  // (4mt + 2(n/16) + (j%4)/2) ^ 4(j/4): one register per mt, the block and
  // group enter as row offsets.
  uint32_t v_rd[4];
  {
    const int j = n & 15;
    const int q = j >> 2;
    const uint32_t base = (uint32_t)((16 * h + q) * kRowBytes + 8 * (j & 1));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      v_rd[mt] = base + 16u * (uint32_t)((4 * mt + 2 * (n >> 4) + ((j & 3) >> 1)) ^ (4 * q));
  }

  const int bs_log2 = P.bs_log2;
  const int bs_mask = P.bs - 1;
  const int64_t head_bytes = (int64_t)g * kD * 2;
  const int32_t* __restrict__ bt_row = block_table + (int64_t)b * P.max_blocks;
  const uint32_t last_page = (uint32_t)((L > 0 ? L : 1) - 1) >> bs_log2;
  // raw page-table entry of this wave's keys of the sub-tile at j0 (a
  // scalar load; keys past L map to the request's last page)
  auto page_of = [&](int j0) -> int {
    uint32_t pidx = (uint32_t)(j0 + 4 * wave) >> bs_log2;
    pidx = pidx > last_page ? last_page : pidx;
    return bt_row[pidx];
  };
  // caches under 4 GB: one resource each, a copy passes its page's offset
  // as the scalar offset (page ids are clamped into the pool first: the
  // scalar offset is outside the resource's range check)
  const u32x4_t k_rsrc = make_rsrc(P.k, 0xffffffffu);
  const u32x4_t v_rsrc = make_rsrc(P.v, 0xffffffffu);
  const uint32_t page_bytes = (uint32_t)P.bs * row_bytes;
  // byte offset inside a page of this wave's first key of sub-tile j of a
  // tile whose first key is a multiple of 64 (plus the tile's own offset
  // inside the page when pages hold more than 64 keys)
  uint32_t kv_in_page[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    kv_in_page[j] = (uint32_t)((kSub * j + 4 * wave) & bs_mask) * row_bytes + (uint32_t)head_bytes;
  const char* kbytes = reinterpret_cast<const char*>(P.k);
  const char* vbytes = reinterpret_cast<const char*>(P.v);

  // ---- relative-bias copy geometry ----
  // The wave's slice of a tile is, for each of its 32 rows, the 64 entries
  // d = p - j0 - 63 .. p - j0 (128 contiguous bytes) as eight 16-byte
  // pieces: piece q holds d = p - j0 - 63 + 8q .. +7. Pieces 4..7 serve the
  // sub-tile at j0 and pieces 0..3 the one at j0 + 32; in sub-tile j, piece
  // (3 - 2u - h) + 4(1 - j) holds the bias of keys 16u + 8h + 7 - x for entry
  // x. Copy instruction m moves rows 8m .. 8m + 7 whole: lane l takes row
  // r = 8m + l / 8 and lands in its LDS row at slot l % 8, which holds piece
  // (l % 8) ^ ((r / 2) % 8) (the slots of a row are XOR-swizzled so that
  // each 16-lane group of a piece read covers all banks once). One
  // instruction thus reads 8 runs of 128 bytes; its 1 KB lands in lane
  // order.
  // Copies read through one resource over the wave's rows plus 64 entries
  // on each side (inside the tensor). A piece is read from its position
  // clamped into the resource: with E >= 8 a piece moved that way holds an
  // entry in 0 <= d < E only in the first or last row of the tensor, whose
  // lanes shift the entries back into place (rewriting the slice in LDS
  // before the bias is added).
  const int E = P.E;
  const int64_t tensor_elems = (int64_t)P.T * P.H * E;
  int64_t reg_lo = 0, reg_hi = 0;
  {
    const int rw0 = min(r0 + 32 * wave, nrows - 1), rw1 = min(r0 + 32 * wave + 31, nrows - 1);
    const int64_t row_min = (int64_t)(t0 + rw0 / G) * P.H + g * G;
    const int64_t row_max = (int64_t)(t0 + rw1 / G) * P.H + g * G + G - 1;
    reg_lo = row_min * E - 64;
    reg_hi = (row_max + 1) * E + 64;
    reg_lo = reg_lo < 0 ? 0 : reg_lo;
    reg_hi = reg_hi > tensor_elems ? tensor_elems : reg_hi;
    if (E == 0) reg_lo = reg_hi = 0;
  }
  const char* rel_base = E > 0 ? reinterpret_cast<const char*>(P.rel) + reg_lo * 2 : reinterpret_cast<const char*>(P.q);
  const u32x4_t rel_rsrc = make_rsrc(rel_base, (uint32_t)((reg_hi - reg_lo) * 2));
  const int64_t my_row_abs = (int64_t)t * P.H + hq;
  const int rel_lane_elem = (int)(my_row_abs * E - reg_lo);  // row start, relative to the resource
  const int rel_last_piece = (int)(reg_hi - reg_lo) - 8;      // last piece start inside the resource
  const int rel_last_byte = 2 * rel_last_piece;
  // the pieces this lane copies (m = 0..3): byte offset of the piece's first
  // entry for the tile at key 0, relative to the resource; cp_second: the
  // piece serves the second sub-tile
  int cp_byte[4];
  bool cp_second[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int piece = (lane & 7) ^ ((4 * (m & 1) + (lane >> 4)) & 7);
    cp_second[m] = piece < 4;
    const int rc = min(r0 + 32 * wave + 8 * m + (lane >> 3), nrows - 1);
    const int itok_c = rc / G;
    const int64_t row_abs_c = (int64_t)(t0 + itok_c) * P.H + g * G + rc % G;
    cp_byte[m] = 2 * ((int)(row_abs_c * E - reg_lo) + (itok_c + L - S) - 63 + 8 * piece);
  }
  // where lane (h, n) finds piece u of sub-tile j of its row
  uint32_t bias_rd[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      bias_rd[j][u] = (uint32_t)(1024 * (n >> 3) + 128 * (n & 7) + 16 * (((3 - 2 * u - h) + 4 * (1 - j)) ^ ((n >> 1) & 7)));
  const bool edge_row = E > 0 && row_ok && (my_row_abs == 0 || my_row_abs == (int64_t)P.T * P.H - 1);
  // distances covered by a sub-tile over the workgroup's rows: [p_lo - j0 - 31, p_hi - j0]
  const int p_lo = ia + L - S, p_hi = ib + L - S;
  // sub-tile at j0 -> 0: no key gets a bias, 1: every score does, 2: some
  // do; as thresholds on j0: none when j0 <= band_a (every distance >= E) or
  // j0 > band_d (every distance < 0), all when band_b < j0 <= band_c
  const int band_a = E == 0 ? 0x7fffffff : p_lo - (kSub - 1) - E;
  const int band_b = p_hi - E, band_c = p_lo - (kSub - 1), band_d = p_hi;
  auto band_class = [&](int j0) -> int {
    const int js = __builtin_amdgcn_readfirstlane(j0);
    const bool none = (js <= band_a) | (js > band_d);
    const bool all = (js > band_b) & (js <= band_c);
    return none ? 0 : (all ? 1 : 2);
  };
  // A operand of the bias MFMAs: lane (h', m) holds row m (key sigma(m)) and
  // k slots 8h' + x; slot x of part u stands for key 16u + 8h' + 7 - x; the
  // entry is the selection value (1/scale or 1) where that key is sigma(m),
  // else 0.
  u32x4_t bias_sel[2];
  {
    const int m = n;
    const int sig = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
    const uint32_t cbits = kExactSel ? (pack_bf16x2(inv_scale, 0.f) & 0xffffu) : 0x3f80u;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int x = 16 * u + 8 * h + 7 - sig;  // slot that matches, if in 0..7
      u32x4_t v = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (x == e) v[e >> 1] = (e & 1) ? (cbits << 16) : cbits;
      bias_sel[u] = v;
    }
  }

  // K/V copies of sub-tile j of the tile in kv whose first key is j0 (a
  // multiple of 64)
  auto issue_kv = [&](char* kv, int j, int j0, int page) {
    page = page < 0 ? 0 : (page >= P.num_blocks ? P.num_blocks - 1 : page);
    page = __builtin_amdgcn_readfirstlane(page);
    if constexpr (kWide) {
      const int key0 = j0 + kSub * j + 4 * wave;
      const int64_t base = (((int64_t)page << bs_log2) + (key0 & bs_mask)) * row_bytes + head_bytes;
      dma16(make_rsrc(kbytes + base, 0x7fffffffu), kv + kSubBytes * j + k_dst, k_src);
      dma16(make_rsrc(vbytes + base, 0x7fffffffu), kv + kSubBytes * j + v_dst, v_src);
    } else {
      const uint32_t off = __builtin_amdgcn_readfirstlane((uint32_t)page * page_bytes + kv_in_page[j] +
                                                          (uint32_t)(j0 & bs_mask) * row_bytes);
      dma16_soff(k_rsrc, kv + kSubBytes * j + k_dst, k_src, off);
      dma16_soff(v_rsrc, kv + kSubBytes * j + v_dst, v_src, off);
    }
  };
  // bias copies of the tile at j0 into bias (the wave's slice); the pieces
  // of a sub-tile that no bias reaches read at an offset past the resource's
  // range, which returns zeros without touching memory, so that they hold
  // zeros
  // (copy instructions m_lo .. m_hi - 1 of the four; none0 / none1: the
  // first / second sub-tile is outside the band)
  auto issue_bias_nn = [&](char* my_bias, int j0, bool none0, bool none1, int m_lo, int m_hi) {
    if (!(none0 | none1)) {
      // both sub-tiles reach the band (the common case)
#pragma unroll
      for (int m = m_lo; m < m_hi; ++m) dma16(rel_rsrc, my_bias + 1024 * m, clamp0(cp_byte[m] - 2 * j0, rel_last_byte));
    } else {
#pragma unroll
      for (int m = m_lo; m < m_hi; ++m)
        dma16(rel_rsrc, my_bias + 1024 * m,
              (cp_second[m] ? none1 : none0) ? kOutOfRange : clamp0(cp_byte[m] - 2 * j0, rel_last_byte));
    }
  };
  auto issue_bias = [&](char* my_bias, int j0, int m_lo = 0, int m_hi = 4) {
    issue_bias_nn(my_bias, j0, band_class(j0) == 0, band_class(j0 + kSub) == 0, m_lo, m_hi);
  };

  f32x16_t oacc[kD / 32];  // O^T: dim tile mt, lane (h, n) reg a = dim 32mt + 8(a/4) + 4h + a%4
#pragma unroll
  for (int mt = 0; mt < kD / 32; ++mt)
#pragma unroll
    for (int a = 0; a < 16; ++a) oacc[mt][a] = 0.f;
  float m_ref = kNegInf;  // running reference max of the column (log2 units)
  float l_part = 0.f;     // this lane's share of the column sum
  const float scale_log2 = P.scale_log2;  // scores are acc * scale_log2 (bias included)
  const bool edge_wave = __builtin_amdgcn_ballot_w64(edge_row) != 0;

  // S^T += K Q^T for both sub-tiles of the tile in kv: register a of lane
  // (h, n) is key j0 + 16h + a; the two MFMA chains interleaved (a chain's
  // next step waits for its previous one)
  auto qk2 = [&](const char* kv, f32x16_t* s) {
    // K operand reads run two steps ahead of the matrix instructions (order
    // pinned with scheduling barriers)
    u32x4_t kf[3][2];
    auto load = [&](int kk) {
#pragma unroll
      for (int j = 0; j < 2; ++j) kf[kk % 3][j] = *reinterpret_cast<const u32x4_t*>(kv + kSubBytes * j + k_rd[kk]);
    };
    load(0);
    load(1);
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      if (kk + 2 < kD / 16) load(kk + 2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v_t, kf[kk % 3][j]),
                                                       __builtin_bit_cast(bf16x8v_t, qreg[kk]), s[j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The start of the score accumulator of the sub-tile at j0: bias / scale,
  // by two MFMAs (and, when the selection value is 1 and the band reaches
  // the sub-tile, an fp32 multiply); outside the band the slice holds zeros
  // and so does the result. Two rare cases first rewrite
  // the wave's slice in LDS (in branches that leave no values behind, so
  // that the common path reads the slice as it is): where the band covers
  // part of the tile, entries outside it are zeroed; in waves holding the
  // first or last row of rel_logits, pieces read at a clamped position are
  // shifted back into place.
  auto bias_acc = [&](char* my_bias, int j, int j0, int bc, f32x16_t& s) {
    if (bc == 2 || (bc == 1 && edge_wave)) {
      asm volatile("");
      // piece u: entry x is distance e_lo0 - 16u + x (key 16u + 8h + 7 - x)
      const int e_lo0 = p - (j0 + 8 * h) - 7;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4_t v = *reinterpret_cast<const u32x4_t*>(my_bias + bias_rd[j][u]);
        if (edge_wave) {
          // a piece read at `at` instead of `want` has its entries moved
          // back by want - at
          const int want = rel_lane_elem + e_lo0 - 16 * u;
          const int at = min(max(want, 0), rel_last_piece);
          v = shift_entries(v, want - at);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int e = e_lo0 - 16 * u + 2 * w;
          const uint32_t lo_ok = (uint32_t)e < (uint32_t)E ? 0xffffu : 0u;
          const uint32_t hi_ok = (uint32_t)(e + 1) < (uint32_t)E ? 0xffff0000u : 0u;
          v[w] &= lo_ok | hi_ok;
        }
        *reinterpret_cast<u32x4_t*>(my_bias + bias_rd[j][u]) = v;
      }
      // the common path below reloads the slice
      asm volatile("" ::: "memory");
    }
    u32x4_t bb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) bb[u] = *reinterpret_cast<const u32x4_t*>(my_bias + bias_rd[j][u]);
    const f32x16_t zero = {};
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v_t, bias_sel[0]),
                                                __builtin_bit_cast(bf16x8v_t, bb[0]), zero, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v_t, bias_sel[1]),
                                                __builtin_bit_cast(bf16x8v_t, bb[1]), s, 0, 0, 0);
    if constexpr (!kExactSel) {
      if (bc != 0) {
#pragma unroll
        for (int a = 0; a < 16; ++a) s[a] *= inv_scale;
      }
    }
  };
  // scores of keys a row does not see -> -inf (only on tiles some row does
  // not see whole)
  auto mask_scores = [&](int j0, f32x16_t* s) {
    const bool interior = (j0 >= lo_max) && (j0 + kKeys <= hi_min);
    if (!interior) {
      asm volatile("");
      // visible registers of sub-tile j: row_lo - jb <= a < row_hi - jb
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int jb = j0 + kSub * j + 16 * h;
        const int a_lo = row_lo - jb, a_hi = row_hi - jb;
#pragma unroll
        for (int a = 0; a < 16; ++a) s[j][a] = (a >= a_lo && a < a_hi) ? s[j][a] : kNegInf;
      }
    }
  };
  // O^T += V^T P^T for sub-tile j of the tile in kv; pb holds P^T (bf16) as
  // the B operand: block kb is registers 8kb..8kb+7 of the sub-tile's scores
  auto pv = [&](const char* kv, int j, const u32x4_t* pb) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int mt = 0; mt < kD / 32; ++mt) {
        u32x2_t part[2];
#pragma unroll
        for (int sr = 0; sr < 2; ++sr) {
          const char* addr = kv + kHalf + kSubBytes * j + (8 * kb + 4 * sr) * kRowBytes + v_rd[mt];
          part[sr] = __builtin_bit_cast(
              u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)addr));
        }
        const u32x4_t av = {part[0][0], part[0][1], part[1][0], part[1][1]};
        oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v_t, av),
                                                           __builtin_bit_cast(bf16x8v_t, pb[kb]), oacc[mt], 0, 0, 0);
      }
  };

  // The tile holding key L - 1 may hold keys past L, whose V rows may be
  // anything (NaN) while their probabilities are 0 (0 * NaN = NaN): once it
  // is in LDS the workgroup overwrites those rows with zeros. Thread i
  // clears 16 bytes of rows i/16 and 32 + i/16.
  auto zero_v_tail = [&](char* kv, int j0) {
    const int r_from = L - j0;  // rows r_from .. 63 hold keys past L
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = (threadIdx.x >> 4) + 32 * rr;
      if (r >= r_from) *reinterpret_cast<u32x4_t*>(kv + kHalf + r * kRowBytes + 16 * (threadIdx.x & 15)) = u32x4_t{0u, 0u, 0u, 0u};
    }
    // the stores have landed before the barrier (lgkmcnt(0) only)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
    lds_barrier();
  };

  // ---- key loop ----
  // Rings in LDS: the K/V tile is copied one tile ahead (2 slots), the bias
  // slices two tiles ahead (3 slots; the bias stream has no reuse and comes
  // from HBM); page ids are loaded a stage before the copy that uses them.
  // Stage s waits for the wave's own copies of tile s, i.e. until only the 4
  // bias copies of tile s + 1 are outstanding, then meets the other waves at
  // a barrier without a memory fence (a fence would wait for every copy in
  // flight). Past the barrier every wave is done with tile s - 1, whose
  // slots then take the K/V of tile s + 1 and the bias of tile s + 2. Copies
  // past the last tile re-read it, so that every stage issues the same
  // copies.
  if (tile_begin < tile_end) {
    const int tb = tile_begin, te = tile_end;
    const int last = te - 1;
    auto j0_of = [&](int it) { return kstart + kKeys * min(it, last); };
    auto kv_slot = [&](int i) { return kv_buf + i * kKV; };
    auto b_slot = [&](int i) { return bias_buf + i * (kWaves * kBiasWave) + wave * kBiasWave; };
    auto issue_bias_tile = [&](int slot, int j0) { issue_bias(b_slot(slot), j0); };
    // copies of the stages before tb: bias tb, K/V tb, bias tb + 1
    issue_bias_tile(0, j0_of(tb));
    issue_kv(kv_slot(0), 0, j0_of(tb), page_of(j0_of(tb)));
    issue_kv(kv_slot(0), 1, j0_of(tb), page_of(j0_of(tb) + kSub));
    issue_bias_tile(1, j0_of(tb + 1));
    int page_next0 = page_of(j0_of(tb + 1)), page_next1 = page_of(j0_of(tb + 1) + kSub);
    // one stage; the slots of tile s (K/V: KVI, bias: BI) are constants of
    // the instance, so that LDS addresses take immediate offsets
    auto stage = [&](int s, auto kvi_c, auto bi_c) {
      constexpr int kv_i = decltype(kvi_c)::value;
      constexpr int b_i = decltype(bi_c)::value;
      wait_vm<4>();
      lds_barrier();
      // the page ids are used only from here on, so that the wait for
      // their loads comes after the long wait above
      int page0 = page_next0, page1 = page_next1;
      asm volatile("" : "+s"(page0), "+s"(page1));
      const int j0 = j0_of(s);
      const int jn = j0_of(s + 1);
      const int j2 = j0_of(s + 2);
      constexpr int b_n = b_i == 0 ? 2 : b_i - 1;  // slot of tile s - 1 = slot of tile s + 2
      page_next0 = page_of(j2);
      page_next1 = page_of(j2 + kSub);
      char* kv = kv_slot(kv_i);
      if (j0 + kKeys > L) zero_v_tail(kv, j0);
      // S^T = bias / scale + K Q^T of the two sub-tiles. The copies of later
      // tiles (K/V of tile s + 1, then the bias of tile s + 2, in that order
      // as the waits assume) are spread over the stage instead of leaving
      // together after the barrier, so that the vector memory path takes
      // them while the stage computes (measured: 3% faster). The band classes
      // of the sub-tiles computed and copied are taken once per stage.
      const int bc0 = band_class(j0), bc1 = band_class(j0 + kSub);
      const bool nn0 = band_class(j2) == 0, nn1 = band_class(j2 + kSub) == 0;
      f32x16_t sc[2];
      bias_acc(b_slot(b_i), 0, j0, bc0, sc[0]);
      issue_kv(kv_slot(kv_i ^ 1), 0, jn, page0);
      bias_acc(b_slot(b_i), 1, j0 + kSub, bc1, sc[1]);
      issue_kv(kv_slot(kv_i ^ 1), 1, jn, page1);
      qk2(kv, sc);
      issue_bias_nn(b_slot(b_n), j2, nn0, nn1, 0, 2);
      mask_scores(j0, sc);
      // row max of the unscaled scores, scaled (log2 units); a new reference
      // only when it grows by more than the slack
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sc[j][a]);
      mx = row_ok ? mx * scale_log2 : kNegInf;
      mx = lane_swap32_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleSlack) != 0) {
        asm volatile("");
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = m_ref == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        l_part *= alpha;
#pragma unroll
        for (int mt = 0; mt < kD / 32; ++mt) oacc[mt] *= alpha;
      }
      const float m_use = m_ref == kNegInf ? 0.f : m_ref;
      // probabilities (bf16) and their sum, then O += P V per sub-tile
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4_t pb[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float e[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) e[x] = __builtin_amdgcn_exp2f(fmaf(sc[j][8 * kb + x], scale_log2, -m_use));
          pb[kb] = u32x4_t{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
#pragma unroll
          for (int w = 0; w < 4; ++w) l_part = dot2_bf16_ones(pb[kb][w], l_part);
        }
        pv(kv, j, pb);
        if (j == 0) issue_bias_nn(b_slot(b_n), j2, nn0, nn1, 2, 4);
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // six stages cover every (K/V slot, bias slot) pair once
    int s = tb;
    for (; s + 6 <= te; s += 6) {
      stage(s, I0{}, I0{});
      stage(s + 1, I1{}, I1{});
      stage(s + 2, I0{}, I2{});
      stage(s + 3, I1{}, I0{});
      stage(s + 4, I0{}, I1{});
      stage(s + 5, I1{}, I2{});
    }
    const int rem = te - s;
    if (rem > 0) stage(s, I0{}, I0{});
    if (rem > 1) stage(s + 1, I1{}, I1{});
    if (rem > 2) stage(s + 2, I0{}, I2{});
    if (rem > 3) stage(s + 3, I1{}, I0{});
    if (rem > 4) stage(s + 4, I0{}, I1{});
    // the last copies re-read tiles nobody uses: let them land before the
    // LDS is released
    __builtin_amdgcn_s_waitcnt(0);
  }

  // ---- epilogue: normalise and write this lane's column ----
  const float l_tot = lane_swap32_sum(l_part);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (P.splits == 1) {
    uint16_t* op = reinterpret_cast<uint16_t*>(P.out) + ((int64_t)t * P.H + hq) * kD;
#pragma unroll
    for (int mt = 0; mt < kD / 32; ++mt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * mt + 8 * a4 + 4 * h;
        u32x2_t w = {pack_bf16x2(oacc[mt][4 * a4] * inv, oacc[mt][4 * a4 + 1] * inv),
                     pack_bf16x2(oacc[mt][4 * a4 + 2] * inv, oacc[mt][4 * a4 + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(op + d0) = w;
      }
  } else {
    const int64_t slotw = ((int64_t)split * P.T + t) * P.H + hq;
    float* wo = P.ws_o + slotw * kD;
#pragma unroll
    for (int mt = 0; mt < kD / 32; ++mt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * mt + 8 * a4 + 4 * h;
        *reinterpret_cast<f32x4_t*>(wo + d0) =
            f32x4_t{oacc[mt][4 * a4] * inv, oacc[mt][4 * a4 + 1] * inv, oacc[mt][4 * a4 + 2] * inv, oacc[mt][4 * a4 + 3] * inv};
      }
    if (h == 0) P.ws_lse[slotw] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

// whether 1/softmax_scale (fp32) is a bf16 number (low 16 bits zero)
static bool inv_scale_is_bf16(float inv) {
  uint32_t u;
  __builtin_memcpy(&u, &inv, 4);
  return (u & 0xffffu) == 0u;
}

bool prefill_supported(const AttnParams& P, int dtype_bf16, int head_dim) {
  // resource offsets are 32-bit: the bias rows of one wave must span less
  // than 2 GB (E * H * (32/G + 2) entries)
  const int64_t span = (int64_t)P.E * P.H * (32 / P.G + 2) * 2 + 256;
  // the scores stay unscaled until the exponent: the scale must be positive,
  // with a finite reciprocal
  const float inv = P.scale_log2 > 0.f ? kLog2e / P.scale_log2 : 0.f;
  return dtype_bf16 && head_dim == kD && P.bs_log2 >= 4 && span < 0x7fffffff && P.scale_log2 > 0.f &&
         inv > 0.f && inv < 3.0e38f && (P.E == 0 || P.E >= 8);
}

int launch_prefill(const AttnParams& P, hipStream_t stream) {
  const int qtiles = (P.max_q * P.G + kRowsWG - 1) / kRowsWG;
  dim3 grid(qtiles * P.splits, P.Hkv, P.B);
  if (grid.x == 0 || P.B == 0) return 0;
  // byte offsets of K/V copies within a cache (a copy reaches up to 4 rows
  // past its first key's row)
  const uint64_t row = (uint64_t)P.Hkv * kD * 2;
  const uint64_t cache_bytes = (uint64_t)P.num_blocks * ((uint64_t)1 << P.bs_log2) * row;
  const bool wide = cache_bytes + 4 * row >= ((uint64_t)1 << 32);
  // 1/softmax_scale from the scale in log2 units (softmax_scale * log2 e)
  const float inv_scale = kLog2e / P.scale_log2;
  const bool exact = inv_scale_is_bf16(inv_scale);
  const dim3 block(kWaves * 64);
  if (!wide && exact)
    hipLaunchKernelGGL((attn_prefill_kernel<false, true>), grid, block, 0, stream, P, P.block_table, inv_scale);
  else if (!wide)
    hipLaunchKernelGGL((attn_prefill_kernel<false, false>), grid, block, 0, stream, P, P.block_table, inv_scale);
  else if (exact)
    hipLaunchKernelGGL((attn_prefill_kernel<true, true>), grid, block, 0, stream, P, P.block_table, inv_scale);
  else
    hipLaunchKernelGGL((attn_prefill_kernel<true, false>), grid, block, 0, stream, P, P.block_table, inv_scale);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace relattn
