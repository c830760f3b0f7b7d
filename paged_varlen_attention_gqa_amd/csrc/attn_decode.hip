// Decode attention kernel: requests whose packed query rows (S_b * G) fit in
// one 16-column MFMA tile, bf16, head_dim 128, block_size a power of two that
// is a multiple of 16.
//
// Each wave owns one (request, KV head, split) and streams the split's
// 16-key tiles on its own; the NW waves of a workgroup take NW neighbouring
// KV heads of the same (request, split), so together they read NW * 256
// contiguous bytes of every cache slot row. Each wave has a private ring of
// RING tile slots in LDS that buffer loads fill directly (global -> LDS, no
// registers), RING - 1 tiles ahead of the arithmetic. Per tile a wave:
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
// Three launches share that per-wave loop: one workgroup per (request,
// split, group of KV heads); a balanced split of the batch's tiles over one
// round of workgroups (split calls of at most 64 requests; 8 waves with
// progress-balanced issue priorities when the KV head count allows); and, for calls
// with one split (sliding-window calls get one) and few (request, KV head)
// pairs, a workgroup per pair whose waves share its key range and merge
// their partial results in LDS, so that long ranges fill the device without
// a workspace.
//
// Score and bias rule: prhub.com.cn report on vLLM PR #48858, "key source
// snippets" (score_mod_rel_bias); paged-cache layout and the split count:
// docs.vllm.ai inkling_fa4_rel_attention / inkling_fa4_num_splits.
#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace relattn {

namespace {

constexpr int kD = 128;
constexpr int kTile = 16;
constexpr int kRowBytes = kD * 2;              // one key row of K or V in LDS
constexpr int kHalfSlot = kTile * kRowBytes;   // K (or V) part of a slot: 4 KB
constexpr int kBiasOff = 2 * kHalfSlot;        // bias part of a slot: 16 B per lane
constexpr int kSlotBytes = kBiasOff + 64 * 16;  // one tile: K, V, bias; 9 KB
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
constexpr int kDecodeWaves = REL_ATTN_DECODE_WAVES;
constexpr int kDecodeRing = REL_ATTN_DECODE_RING;
// The balanced kernel takes 8 waves (8 KV heads, one workgroup per compute
// unit) when the KV head count is a multiple of 8: waves w and w + 4 then
// share a SIMD, and the one that has computed fewer tiles raises its issue
// priority (on a SIMD the older wave otherwise wins every issue race, and
// the younger one finishes about 30% later; measured: 3% less time in all).
// Other head counts take 4-wave workgroups, two per compute unit.
constexpr int kBalancedWaves = 8;
// in-workgroup split of one-split calls: waves per (request, KV head), and
// when it is used (fewer pairs than this, key ranges of at least this many
// keys: each wave then streams at least 4 tiles)
constexpr int kWgSplitWaves = 4;
constexpr int kWgSplitMaxPairs = 1024;
constexpr int kWgSplitMinKeys = 4 * kWgSplitWaves * 16;

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
// [16l, 16l+16) of the destination block. The copies carry the non-temporal
// cache policy (the nt bit of the instruction's cache-policy field): every
// K/V row is read once, and streaming it past the caches lets the loads
// return sooner (measured: about 10% more bandwidth).
constexpr int kStreamPolicy = 2;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 16, voff, 0, 0, kStreamPolicy);
}

// Where a wave of the in-workgroup split leaves its partial result: its
// own two ring slots, once its copies have landed (o: 16 columns x 128 dims
// fp32 in the first, one log2-sum-exp per column in the second).
struct LdsPartial {
  float* o;
  float* lse;
};

// One wave's work on one piece of one request: the request's rows (S * G
// <= 16 columns) against KV head g over the keys [c0, c1) (c0 a multiple of
// 16 inside the request's visible range, c1 its end or a later multiple of
// 16), written to `out` when the call has one split, else to split slot
// `split` of the workspace (normalised partial output and log-sum-exp).
// block_table is the same table as P.block_table, restrict-qualified so that
// page lookups compile to scalar loads: they then count on the scalar/LDS
// counter and a wait for them never waits for the K/V copies in flight.
template <int NW, int RING, bool PART = false, bool BAL = false>
__device__ __forceinline__ void decode_piece(const AttnParams& P, const int32_t* __restrict__ block_table,
                                             char* ring0, char* ring1, char* ring2, int wave, int lane,
                                             int b, int g, int t0, int S, int L, int c0_in, int c1_in,
                                             int split, LdsPartial part = {nullptr, nullptr},
                                             int* prog = nullptr) {
  const int n = lane & 15;  // column (query row) / K row / transpose-read lane
  const int q = lane >> 4;  // 0..3
  const int G = P.G;
  const int rows = S * G;

  // column n: token n / G of the request, query head g*G + n % G
  const bool col_ok = n < rows;
  const int itok = col_ok ? n / G : 0;
  const int hh = col_ok ? n % G : 0;
  const int h = g * G + hh;
  const int t = t0 + itok;
  const int p = itok + L - S;
  int row_lo = 0, row_hi = 0;
  if (col_ok) visible_range(P, p, L, row_lo, row_hi);

  const int c0 = __builtin_amdgcn_readfirstlane(c0_in);
  const int c1 = __builtin_amdgcn_readfirstlane(c1_in);
  const int ntiles = __builtin_amdgcn_readfirstlane(c1 > c0 ? (c1 - c0 + kTile - 1) / kTile : 0);

  if (ntiles == 0) {
    // No visible key: the row's output is zero, and an empty split still
    // tells the combine step that it holds nothing. Lane (n, q) writes dims
    // 32q .. 32q+31 of column n.
    if constexpr (PART) {
      if (q == 0) part.lse[n] = kNegInf;
      return;
    }
    if (col_ok) {
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

  // relative-bias rows of this wave's columns: one resource from the first
  // column's row, lane offsets relative to it
  const int E = P.E;
  const int Em8 = E >= 8 ? E - 8 : 0;  // last start of 8 entries inside a row
  const char* rel_base = E > 0 ? reinterpret_cast<const char*>(P.rel) + ((int64_t)t0 * P.H + g * G) * E * 2
                               : reinterpret_cast<const char*>(P.q);
  const uint32_t rel_lane = E > 0 ? (uint32_t)((itok * P.H + hh) * E) * 2u : 0u;
  const __amdgpu_buffer_rsrc_t rel_rsrc = make_rsrc(rel_base);

  const int bs_log2 = P.bs_log2;
  const int bs_mask = P.bs - 1;
  const int32_t* __restrict__ bt_row = block_table + (int64_t)b * P.max_blocks;
  const int last_pidx = (c1 - 1) >> bs_log2;  // last page the split reads

  const char* kbytes = reinterpret_cast<const char*>(P.k);
  const char* vbytes = reinterpret_cast<const char*>(P.v);
  const int64_t head_bytes = (int64_t)g * kD * 2;
  char* const my0 = ring0 + wave * kSlotBytes;
  char* const my1 = ring1 + wave * kSlotBytes;
  char* const my2 = ring2 + (RING > 2 ? wave * kSlotBytes : 0);

  // raw page-table entry of the tile at key j0 (a scalar load; pages past
  // the split's last one are clamped to it); issue() clamps the id
  auto page_at = [&](int j0) -> int {
    int pidx = j0 >> bs_log2;
    pidx = pidx > last_pidx ? last_pidx : pidx;
    return bt_row[pidx];
  };

  // The bias of lane (q, n) for the tile at j0: keys j0 + 4q + i (i = 0..3)
  // have distances D - i, D = p - j0 - 4q, i.e. entries D-3 .. D of the
  // column's rel_logits row. The copy moves 8 entries from a start clamped
  // into the row (always in bounds) into the lane's 16 bytes of the slot;
  // entries that the clamp shifted out are outside [0, E) and dropped by the
  // arithmetic.
  auto bias_start = [&](int j0) -> int {
    const int d = p - (j0 + 4 * q) - 3;
    return d < 0 ? 0 : (d > Em8 ? Em8 : d);
  };

  // Page ids are scalar loads issued one or two steps before the copy that
  // uses them; after the loop the prefetched values are consumed, which keeps
  // the compiler from sinking the loads next to their use.
  auto keep = [](int v) { asm volatile("; page %0" ::"s"(v)); };

  // start the copy of the tile at key j0 (raw page-table entry given) into a
  // slot: 4 KB of K, 4 KB of V, 1 KB of bias. Every call issues the same
  // nine copies, so the compiler's wait counts stay exact.
  auto issue = [&](char* slot, int j0, int page) {
    page = page < 0 ? 0 : (page >= P.num_blocks ? P.num_blocks - 1 : page);
    const int64_t base = (((int64_t)page << bs_log2) + (j0 & bs_mask)) * row_bytes + head_bytes;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbytes + base);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbytes + base);
    dma16(rel_rsrc, slot + kBiasOff, rel_lane + 2u * (uint32_t)bias_start(j0));
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

  auto compute = [&](const char* slot, int j0) {
    // S^T = K Q^T
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kD / 32; ++c) {
      const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(slot + k_rd[c]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf),
                                                  __builtin_bit_cast(bf16x8_t, qreg[c]), s, 0, 0, 0);
    }
    // entry of key j0 + 4q + i among the lane's 8 copied ones is sh - i
    const int sh = p - (j0 + 4 * q) - bias_start(j0);
    const uint16_t* my_bias = reinterpret_cast<const uint16_t*>(slot + kBiasOff + 16 * lane);
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * q + i;
      const uint32_t in_range = (uint32_t)(p - j) < (uint32_t)E ? 0xffffffffu : 0u;
      const int k = sh - i < 0 ? 0 : (sh - i > 7 ? 7 : sh - i);
      const uint32_t bits = (uint32_t)my_bias[k] << 16;
      const float bv = __uint_as_float(bits & in_range);
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

  // progress balance of the two waves that share a SIMD (w and w ^ 4):
  // the one that has computed fewer tiles takes issue priority
  auto balance = [&]() {
    if constexpr (BAL) {
      const int mine = __builtin_amdgcn_readfirstlane(prog[wave]) + 1;
      prog[wave] = mine;
      const int other = __builtin_amdgcn_readfirstlane(prog[wave ^ 4]);
      if (mine < other)
        __builtin_amdgcn_s_setprio(2);
      else
        __builtin_amdgcn_s_setprio(0);
    }
  };
  // ---- key loop over the split's tiles; RING-1 tiles in flight ----
  // The loop runs whole iterations only (no exit inside its body): each step
  // copies one tile RING-1 ahead and loads the page id of the tile two
  // steps later still; the remaining tiles are computed after it.
  {
    const int nw = ntiles;
    // tiles past the last (prefetches only) map to the last one: always
    // inside the split's pages
    const int i_max = nw - 1;
    auto j0_of = [&](int i) { return c0 + kTile * (i < i_max ? i : i_max); };
    // Before computing a tile, a wave waits for its own copies of it: until
    // only the copies issued after them (9 per tile) are outstanding. The
    // waits are explicit because the compiler does not see which LDS bytes
    // a buffer-to-LDS copy writes.
    if constexpr (RING == 3) {
      // iteration k: tiles 3k .. 3k+2 computed, 3k+2 .. 3k+4 copied
      if (nw > 0) issue(my0, j0_of(0), page_at(j0_of(0)));
      if (nw > 1) issue(my1, j0_of(1), page_at(j0_of(1)));
      int pa = page_at(j0_of(2)), pb = page_at(j0_of(3)), pc = page_at(j0_of(4));
      const int iters = nw >= 3 ? (nw - 2) / 3 : 0;
      int i = 0;
      for (int k = 0; k < iters; ++k, i += 3) {
        issue(my2, j0_of(i + 2), pa);
        wait_vm<18>();
        compute(my0, j0_of(i));
        // the next iteration's page ids, issued after the compute's LDS
        // reads have been waited for (scalar loads and LDS reads share a
        // counter): they complete before its next wait, which follows the
        // wait for a tile
        __builtin_amdgcn_sched_barrier(0);
        const int na = page_at(j0_of(i + 5)), nb = page_at(j0_of(i + 6)), nc = page_at(j0_of(i + 7));
        issue(my0, j0_of(i + 3), pb);
        wait_vm<18>();
        compute(my1, j0_of(i + 1));
        issue(my1, j0_of(i + 4), pc);
        wait_vm<18>();
        compute(my2, j0_of(i + 2));
        pa = na;
        pb = nb;
        pc = nc;
      }
      keep(pa);
      keep(pb);
      keep(pc);
      // tiles i, i+1 are copied (if they exist); at most two more remain
      if (i + 2 < nw) {
        issue(my2, j0_of(i + 2), pa);
        wait_vm<18>();
        compute(my0, j0_of(i));
        if (i + 3 < nw) {
          issue(my0, j0_of(i + 3), pb);
          wait_vm<18>();
          compute(my1, j0_of(i + 1));
          wait_vm<9>();
          compute(my2, j0_of(i + 2));
          wait_vm<0>();
          compute(my0, j0_of(i + 3));
        } else {
          wait_vm<9>();
          compute(my1, j0_of(i + 1));
          wait_vm<0>();
          compute(my2, j0_of(i + 2));
        }
      } else if (i + 1 < nw) {
        wait_vm<9>();
        compute(my0, j0_of(i));
        wait_vm<0>();
        compute(my1, j0_of(i + 1));
      } else if (i < nw) {
        wait_vm<0>();
        compute(my0, j0_of(i));
      }
    } else {
      // iteration k: tiles 2k, 2k+1 computed, 2k+1, 2k+2 copied
      if (nw > 0) issue(my0, j0_of(0), page_at(j0_of(0)));
      int pa = page_at(j0_of(1)), pb = page_at(j0_of(2));
      const int iters = nw >= 1 ? (nw - 1) / 2 : 0;
      int i = 0;
      for (int k = 0; k < iters; ++k, i += 2) {
        issue(my1, j0_of(i + 1), pa);
        wait_vm<9>();
        compute(my0, j0_of(i));
        balance();
        // the next iteration's page ids, issued after the compute's LDS
        // reads have been waited for (scalar loads and LDS reads share a
        // counter): they complete before its next wait, which follows the
        // wait for a tile
        __builtin_amdgcn_sched_barrier(0);
        const int na = page_at(j0_of(i + 3)), nb = page_at(j0_of(i + 4));
        issue(my0, j0_of(i + 2), pb);
        wait_vm<9>();
        compute(my1, j0_of(i + 1));
        balance();
        pa = na;
        pb = nb;
      }
      keep(pa);
      keep(pb);
      // tile i is copied (if it exists); at most one more remains
      if (i + 1 < nw) {
        issue(my1, j0_of(i + 1), pa);
        wait_vm<9>();
        compute(my0, j0_of(i));
        wait_vm<0>();
        compute(my1, j0_of(i + 1));
      } else if (i < nw) {
        wait_vm<0>();
        compute(my0, j0_of(i));
      }
    }
  }

  // ---- epilogue: normalise and write this wave's columns ----
  // lane (q, n) holds dims 16mb + 4q + i of column n; m_ref is the column's
  // reference max (log2 units), the same in the four lanes of a column
  const float l_col = wave_sum_xor_16_32(l_part);
  if constexpr (PART) {
    // the wave's copies (also the ones past its last tile) have landed
    // before its slots take the partial
    wait_vm<0>();
    const float inv = l_col > 0.f ? 1.f / l_col : 0.f;
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb) *reinterpret_cast<f32x4_t*>(part.o + n * kD + 16 * mb + 4 * q) = oacc[mb] * inv;
    if (q == 0) part.lse[n] = l_col > 0.f ? m_ref + __log2f(l_col) : kNegInf;
    return;
  }
  if (!col_ok) return;
  const float inv = l_col > 0.f ? 1.f / l_col : 0.f;
  if (P.splits == 1) {
    uint16_t* op = reinterpret_cast<uint16_t*>(P.out) + ((int64_t)t * P.H + h) * kD + 4 * q;
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb)
      *reinterpret_cast<u32x2_t*>(op + 16 * mb) =
          u32x2_t{pack_bf16x2(oacc[mb][0] * inv, oacc[mb][1] * inv), pack_bf16x2(oacc[mb][2] * inv, oacc[mb][3] * inv)};
  } else {
    const int64_t slot = ((int64_t)split * P.T + t) * P.H + h;
    float* wo = P.ws_o + slot * kD + 4 * q;
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb) *reinterpret_cast<f32x4_t*>(wo + 16 * mb) = oacc[mb] * inv;
    if (q == 0) P.ws_lse[slot] = l_col > 0.f ? (m_ref + __log2f(l_col)) * kLn2 : kNegInf;
  }
}

// the key range of a request's rows: the union over its first and last
// token, from a multiple of 16 (kstart) to hi; ntiles 16-key tiles
__device__ __forceinline__ void request_keys(const AttnParams& P, int S, int L, int& kstart, int& hi, int& ntiles) {
  int lo_a, hi_a, lo_b, hi_b;
  visible_range(P, L - S, L, lo_a, hi_a);
  visible_range(P, L - 1, L, lo_b, hi_b);
  const int lo = min(lo_a, lo_b);
  hi = max(hi_a, hi_b);
  kstart = lo & ~(kTile - 1);
  ntiles = hi > lo ? (hi - kstart + kTile - 1) / kTile : 0;
}

// One workgroup per (KV head group of NW heads, split, request): split s of
// request b covers the keys [kstart + s * dec_chunk, + dec_chunk).
template <int NW, int RING>
__global__ __launch_bounds__(NW * 64) void attn_decode_kernel(AttnParams P,
                                                              const int32_t* __restrict__ block_table) {
  // One LDS object per ring slot, so that the compiler keeps them apart;
  // wave w owns bytes [w * kSlotBytes, (w + 1) * kSlotBytes) of each.
  __shared__ __attribute__((aligned(1024))) char ring0[NW * kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[NW * kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[RING > 2 ? NW * kSlotBytes : 16];
  static_assert(RING == 2 || RING == 3, "ring depth");
  // wave index as a scalar, so that the tile loop runs on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.z;
  const int split = blockIdx.y;
  const int g = blockIdx.x * NW + wave;  // KV head of this wave
  if (g >= P.Hkv) return;
  int t0, S, L;
  if (!request_bounds(P, b, t0, S, L)) return;
  if (S * P.G > 16) return;  // handled by the prefill or general kernel
  int kstart, hi, ntiles;
  request_keys(P, S, L, kstart, hi, ntiles);
  const int c0 = kstart + split * P.dec_chunk;
  decode_piece<NW, RING>(P, block_table, ring0, ring1, ring2, wave, lane, b, g, t0, S, L, c0,
                         min(c0 + P.dec_chunk, hi), split);
}

// Calls with one split and few (request, KV head) pairs: a workgroup per
// (KV head, request) whose NW waves cut the request's key range into NW
// pieces of whole tiles, then merge their partials through LDS (the split
// of the key range happens inside the workgroup, so it needs no workspace).
template <int NW, int RING>
__global__ __launch_bounds__(NW * 64) void attn_decode_wg_split_kernel(AttnParams P,
                                                                       const int32_t* __restrict__ block_table) {
  __shared__ __attribute__((aligned(1024))) char ring0[NW * kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[NW * kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[RING > 2 ? NW * kSlotBytes : 16];
  static_assert(RING == 2 || RING == 3, "ring depth");
  static_assert(16 * kD * 4 <= kSlotBytes, "a partial fits in a slot");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x;
  const int b = blockIdx.z;
  int t0, S, L;
  if (!request_bounds(P, b, t0, S, L)) return;
  const int rows = S * P.G;
  if (rows > 16) return;  // handled by the prefill or general kernel
  int kstart, hi, ntiles;
  request_keys(P, S, L, kstart, hi, ntiles);
  const int per = (ntiles + NW - 1) / NW;  // tiles per wave
  const int c0 = kstart + kTile * min(wave * per, ntiles);
  const int c1 = min(kstart + kTile * min((wave + 1) * per, ntiles), hi);
  LdsPartial part = {reinterpret_cast<float*>(ring0 + wave * kSlotBytes),
                     reinterpret_cast<float*>(ring1 + wave * kSlotBytes)};
  decode_piece<NW, RING, true>(P, block_table, ring0, ring1, ring2, wave, lane, b, g, t0, S, L, c0,
                               max(c0, c1), 0, part);
  __syncthreads();
  // merge: item i is column i / 32, dims 4 (i % 32) .. + 3
  for (int it = threadIdx.x; it < rows * 32; it += NW * 64) {
    const int col = it >> 5;
    const int d0 = 4 * (it & 31);
    float lse[NW];
    float mmax = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lse[w] = reinterpret_cast<const float*>(ring1 + w * kSlotBytes)[col];
      mmax = fmaxf(mmax, lse[w]);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (mmax != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (lse[w] == kNegInf) continue;
        const float wt = __builtin_amdgcn_exp2f(lse[w] - mmax);
        wsum += wt;
        acc += wt * *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(ring0 + w * kSlotBytes) + col * kD + d0);
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const int t = t0 + col / P.G;
    const int h = g * P.G + col % P.G;
    uint16_t* op = reinterpret_cast<uint16_t*>(P.out) + ((int64_t)t * P.H + h) * kD + d0;
    *reinterpret_cast<u32x2_t*>(op) = u32x2_t{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  }
}

// Balanced split of the whole batch (at most 64 requests, num_splits >= 2):
// the decode-shaped requests' 16-key tiles are laid end to end (N of them)
// and workgroup m of a KV head group takes tiles [m N / M, (m+1) N / M), M
// the number of workgroups used, so every workgroup streams the same number
// of tiles whatever the lengths. A request's tiles then fall to consecutive
// workgroups; the piece of the k-th of them goes to split slot k. M is the
// largest launched count for which no request has more than num_splits
// pieces. Slots a request does not use get lse = -inf.
template <int NW, int RING, int HALVES>
__global__ __launch_bounds__(NW * 64) void attn_decode_balanced_kernel(AttnParams P,
                                                                       const int32_t* __restrict__ block_table) {
  __shared__ __attribute__((aligned(1024))) char ring0[NW * kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[NW * kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[RING > 2 ? NW * kSlotBytes : 16];
  static_assert(RING == 2 || RING == 3, "ring depth");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  __shared__ int prog[NW];
  prog[wave] = 0;
  // HALVES = 2: the workgroup serves NW / 2 heads with two waves each; wave
  // w takes the second half of the workgroup's share when w >= NW / 2 (a
  // workgroup then counts as two of the M workgroups that share the tiles)
  constexpr int kHeads = NW / HALVES;
  const int m = blockIdx.x * HALVES + wave / kHeads;
  const int M = gridDim.x * HALVES;
  const int g = blockIdx.y * kHeads + wave % kHeads;  // KV head of this wave
  if (g >= P.Hkv) return;
  const int K = P.splits;

  // lane l describes request l: first row, rows, keys, key range and tiles
  int t0_l = 0, S_l = 0, L_l = 0, ks_l = 0, hi_l = 0, n_l = 0;
  bool dec_l = false;  // a decode-shaped request with rows
  if (lane < P.B) {
    int t0, S, L;
    if (request_bounds(P, lane, t0, S, L) && S * P.G <= 16) {
      dec_l = true;
      t0_l = t0;
      S_l = S;
      L_l = L;
      request_keys(P, S, L, ks_l, hi_l, n_l);
    }
  }
  // prefix sums of the tile counts over the requests
  int incl = n_l;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  const int excl = incl - n_l;
  const int N = __builtin_amdgcn_readlane(incl, 63);
  int nmax = n_l;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) nmax = max(nmax, __shfl_xor(nmax, off));
  nmax = __builtin_amdgcn_readfirstlane(nmax);

  // workgroups used: pieces per request <= ceil((n - 1) / (N / Me)) + 1 <= K
  // when every workgroup gets at least ceil(nmax / (K - 1)) tiles
  int Me = 1;
  if (N > 0) {
    const int qmin = (nmax + K - 2) / (K - 1);
    Me = N / qmin;
    Me = Me < 1 ? 1 : (Me > M ? M : Me);
  }
  if (m >= Me) return;
  const int a_lo = (int)((int64_t)m * N / Me);
  const int a_hi = (int)((int64_t)(m + 1) * N / Me);

  const int n = lane & 15;
  // all K slots (or those after slot k0) of request b get lse = -inf
  auto clear_slots = [&](int bt0, int brows, int k0) {
    if (n < brows) {
      const int t = bt0 + n / P.G;
      const int h = g * P.G + n % P.G;
      for (int k = k0 + (lane >> 4); k < K; k += 4) P.ws_lse[((int64_t)k * P.T + t) * P.H + h] = kNegInf;
    }
  };

  // requests without visible keys: the workgroup whose range holds their
  // position in the tile sequence (the last one for position N) clears them
  {
    const bool mine = dec_l && n_l == 0 && ((excl >= a_lo && excl < a_hi) || (m == Me - 1 && excl >= a_hi));
    uint64_t mask = __builtin_amdgcn_ballot_w64(mine);
    while (mask) {
      const int bb = __builtin_ctzll(mask);
      mask &= mask - 1;
      clear_slots(__builtin_amdgcn_readlane(t0_l, bb), __builtin_amdgcn_readlane(S_l, bb) * P.G, 0);
    }
  }

  // the requests whose tiles meet [a_lo, a_hi), in order
  uint64_t mask = __builtin_amdgcn_ballot_w64(n_l > 0 && incl > a_lo && excl < a_hi);
  while (mask) {
    const int bb = __builtin_ctzll(mask);
    mask &= mask - 1;
    const int bt0 = __builtin_amdgcn_readlane(t0_l, bb);
    const int bS = __builtin_amdgcn_readlane(S_l, bb);
    const int bL = __builtin_amdgcn_readlane(L_l, bb);
    const int bks = __builtin_amdgcn_readlane(ks_l, bb);
    const int bhi = __builtin_amdgcn_readlane(hi_l, bb);
    const int bn = __builtin_amdgcn_readlane(n_l, bb);
    const int bex = __builtin_amdgcn_readlane(excl, bb);
    const int u0 = max(a_lo, bex) - bex;
    const int u1 = min(a_hi, bex + bn) - bex;
    // piece index: workgroups from the one holding the request's first tile
    const int m_first = (int)(((int64_t)(bex + 1) * Me - 1) / N);
    const int k = m - m_first;
    decode_piece<NW, RING, false, (NW == 8)>(P, block_table, ring0, ring1, ring2, wave, lane, bb, g, bt0, bS, bL,
                           bks + kTile * u0, min(bks + kTile * u1, bhi), k, LdsPartial{nullptr, nullptr}, prog);
    if (u1 == bn) clear_slots(bt0, bS * P.G, k + 1);
  }
}

}  // namespace

bool decode_supported(const AttnParams& P, int dtype_bf16, int head_dim) {
  // the 16-byte bias copies need rows of at least 8 entries
  return dtype_bf16 && head_dim == kD && P.bs_log2 >= 4 && (P.E == 0 || P.E >= 8);
}

namespace {

// workgroups of the balanced kernel (NW waves) resident at once on the
// device (all its compute units), queried once per device
template <int NW, int HALVES>
int balanced_slots() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(attn_decode_balanced_kernel<NW, kDecodeRing, HALVES>), NW * 64, 0) !=
      hipSuccess)
    return 0;
  v = cus * per_cu;
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

// one round of balanced workgroups of NW waves (NW / HALVES heads each)
// over the whole device
template <int NW, int HALVES>
int launch_balanced(const AttnParams& P, hipStream_t stream) {
  const int slots = balanced_slots<NW, HALVES>();
  if (slots <= 0) return -1;
  constexpr int kHeads = NW / HALVES;
  const int groups = (P.Hkv + kHeads - 1) / kHeads;
  const int per_group = slots / groups > 0 ? slots / groups : 1;
  hipLaunchKernelGGL((attn_decode_balanced_kernel<NW, kDecodeRing, HALVES>), dim3(per_group, groups),
                     dim3(NW * 64), 0, stream, P, P.block_table);
  return 0;
}

}  // namespace

int launch_decode(const AttnParams& P, int head_dim, hipStream_t stream) {
  (void)head_dim;
  if (P.B == 0) return 0;
  const int groups = (P.Hkv + kDecodeWaves - 1) / kDecodeWaves;
  if (P.splits > 1 && P.B <= 64) {
    // 8 waves: 8 heads, or 4 heads with two waves each; other head counts
    // take two 4-wave workgroups per compute unit
    const int rc = P.Hkv % 8 == 0   ? launch_balanced<kBalancedWaves, 1>(P, stream)
                   : P.Hkv % 4 == 0 ? launch_balanced<kBalancedWaves, 2>(P, stream)
                                    : launch_balanced<kDecodeWaves, 1>(P, stream);
    if (rc != 0) return -1;
  } else if (P.splits == 1 && (int64_t)P.B * P.Hkv < kWgSplitMaxPairs && P.dec_chunk >= kWgSplitMinKeys) {
    // few (request, KV head) pairs with long key ranges and no workspace:
    // the key range of a pair is shared by the waves of its workgroup
    hipLaunchKernelGGL((attn_decode_wg_split_kernel<kWgSplitWaves, 2>), dim3(P.Hkv, 1, P.B),
                       dim3(kWgSplitWaves * 64), 0, stream, P, P.block_table);
  } else {
    // workgroup: kDecodeWaves neighbouring KV heads of one (request, split)
    hipLaunchKernelGGL((attn_decode_kernel<kDecodeWaves, kDecodeRing>), dim3(groups, P.splits, P.B),
                       dim3(kDecodeWaves * 64), 0, stream, P, P.block_table);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace relattn
