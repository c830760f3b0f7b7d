// C ABI of librelattn.so (declared in include/rel_attn.h): host-side argument
// checks, split-count heuristic, workspace sizing and kernel dispatch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>
#include <mutex>

#include "../../include/rel_attn.h"
#include "kernels.h"

using relattn::AttnParams;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Query rows per work unit in the general kernel, and the decode tile.
constexpr int kGeneralRows = 64;
// Workgroups wanted in flight: 4 per compute unit on 256 CUs.
constexpr int kTargetWorkgroups = 1024;
// Fewest keys worth giving one split.
constexpr int kMinKeysPerSplit = 256;
// Decode-shaped calls (one 16-column tile of query rows per KV head): the
// balanced decode kernel cuts the batch's tiles into one round of 512 pieces
// per 4 KV heads on 256 CUs (two 4-wave workgroups per compute unit, or one
// 8-wave workgroup over 8 heads, or over 4 heads in two halves); splits are
// the most pieces one request may be cut into, with room for requests of
// unequal length, and a piece should hold at least 256 keys.
constexpr int kDecodeWorkgroups = 512;
constexpr int kDecodeHeadsPerWorkgroup = 4;
constexpr int kDecodeMinKeysPerPiece = 256;
constexpr int kMaxSplits = 512;

bool supported_head_dim(int d) { return d == 64 || d == 128; }

}  // namespace

extern "C" int rel_attn_num_splits(int is_local, int batch_size, int max_query_len, int num_heads,
                                   int num_kv_heads, int max_kv_len) {
  if (batch_size < 1 || max_query_len < 1 || num_heads < 1 || num_kv_heads < 1 || max_kv_len < 0 ||
      num_heads % num_kv_heads != 0)
    return REL_ATTN_EINVAL;
  if (is_local) return 1;
  const int64_t G = num_heads / num_kv_heads;
  const int64_t rows = (int64_t)max_query_len * G;
  if (rows <= relattn::kDecodeMaxRows) {
    // the workgroups of one KV head group share the batch's tiles evenly; a
    // request of the longest length then spans about (workgroups per group)
    // / batch pieces if all requests were that long; four times that leaves
    // room for shorter neighbours
    const int64_t groups = ((int64_t)num_kv_heads + kDecodeHeadsPerWorkgroup - 1) / kDecodeHeadsPerWorkgroup;
    const int64_t per_group = kDecodeWorkgroups / groups > 0 ? kDecodeWorkgroups / groups : 1;
    int64_t splits = (4 * per_group + batch_size - 1) / batch_size + 2;
    const int64_t by_len = max_kv_len / kDecodeMinKeysPerPiece + 1;
    if (splits > by_len) splits = by_len;
    if (splits > kMaxSplits) splits = kMaxSplits;
    if (splits < 1) splits = 1;
    return (int)splits;
  }
  // Prefill-shaped calls: split long key ranges until the launch has about
  // 4 workgroups per compute unit.
  const int64_t qtiles = (rows + kGeneralRows - 1) / kGeneralRows;
  const int64_t pairs = (int64_t)batch_size * num_kv_heads;
  // (the product of the two counts is taken only when it stays small)
  int64_t splits = 1;
  if (pairs < kTargetWorkgroups && qtiles < kTargetWorkgroups) {
    const int64_t units = pairs * qtiles;
    splits = (kTargetWorkgroups + units - 1) / units;
  }
  const int64_t by_len = max_kv_len / kMinKeysPerSplit;
  if (splits > by_len) splits = by_len;
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits < 1) splits = 1;
  return (int)splits;
}

extern "C" size_t rel_attn_workspace_bytes(int num_splits, int num_tokens, int num_heads, int head_dim) {
  if (num_splits < 1 || num_tokens < 0 || num_heads < 1 || head_dim < 1) return 0;
  if (num_splits == 1) return 0;
  // a size past what size_t holds is reported as SIZE_MAX, which no
  // workspace can match (the call then fails with REL_ATTN_EWORKSPACE)
  size_t n = (size_t)num_splits;
  for (const size_t f : {(size_t)num_tokens, (size_t)num_heads, (size_t)head_dim + 1u, (size_t)4u}) {
    if (f != 0 && n > SIZE_MAX / f) return SIZE_MAX;
    n *= f;
  }
  return n;
}

extern "C" const char* rel_attn_strerror(int code) {
  switch (code) {
    case REL_ATTN_OK: return "success";
    case REL_ATTN_EINVAL: return "invalid argument";
    case REL_ATTN_EUNSUPPORTED: return "unsupported dtype, head_dim, group size or block_size";
    case REL_ATTN_EWORKSPACE: return "workspace missing or too small for num_splits > 1";
    case REL_ATTN_ELAUNCH: return "HIP kernel launch failed";
    default: return "unknown error code";
  }
}

namespace {

// Host-side checks and parameter set-up shared by rel_attn_fwd and
// rel_attn_fwd_splits. Returns REL_ATTN_OK with *launch = true when kernels
// must run, REL_ATTN_OK with *launch = false for a workspace query or an empty
// call, or a negative code.
int prepare(const void* q, const void* key_cache, const void* value_cache, const int32_t* block_table,
            const int32_t* cache_seqlens, const int32_t* cu_seqlens_q, const void* rel_logits, void* out,
            int dtype, int num_tokens, int batch_size, int max_seqlen_q, int max_blocks_per_seq,
            int num_heads, int num_kv_heads, int head_dim, int num_blocks, int block_size, int rel_extent,
            float softmax_scale, int causal, int window_left, int window_right, int num_splits,
            void* workspace, size_t workspace_bytes, size_t* workspace_needed, AttnParams* P_out,
            bool* launch) {
  *launch = false;
  if (num_tokens < 0 || batch_size < 0 || max_seqlen_q < 0 || max_blocks_per_seq < 0 || num_heads < 1 ||
      num_kv_heads < 1 || head_dim < 1 || num_blocks < 0 || block_size < 1 || rel_extent < 0 ||
      window_left < -1 || window_right < -1 || (causal != 0 && causal != 1))
    return REL_ATTN_EINVAL;
  if (num_heads % num_kv_heads != 0) return REL_ATTN_EINVAL;
  if (num_splits < 1 || num_splits > kMaxSplits) return REL_ATTN_EINVAL;
  if (!(softmax_scale == softmax_scale)) return REL_ATTN_EINVAL;  // NaN scale
  if (dtype != REL_ATTN_FP32 && dtype != REL_ATTN_BF16) return REL_ATTN_EUNSUPPORTED;
  if (!supported_head_dim(head_dim)) return REL_ATTN_EUNSUPPORTED;
  const int G = num_heads / num_kv_heads;
  if (G > 16) return REL_ATTN_EUNSUPPORTED;

  const size_t need = rel_attn_workspace_bytes(num_splits, num_tokens, num_heads, head_dim);
  if (workspace_needed) *workspace_needed = need;
  if (workspace == nullptr && workspace_needed != nullptr) return REL_ATTN_OK;  // size query

  if (batch_size > 0 && (cache_seqlens == nullptr || cu_seqlens_q == nullptr)) return REL_ATTN_EINVAL;
  if (num_tokens > 0 && (q == nullptr || out == nullptr)) return REL_ATTN_EINVAL;
  if (batch_size > 0 && num_tokens > 0 &&
      (key_cache == nullptr || value_cache == nullptr || block_table == nullptr || num_blocks < 1 ||
       max_blocks_per_seq < 1))
    return REL_ATTN_EINVAL;
  if (rel_extent > 0 && num_tokens > 0 && rel_logits == nullptr) return REL_ATTN_EINVAL;
  if (batch_size > 65535 || num_kv_heads > 65535) return REL_ATTN_EUNSUPPORTED;
  if (num_splits > 1 && need > 0) {
    if (workspace == nullptr || workspace_bytes < need || need == SIZE_MAX) return REL_ATTN_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return REL_ATTN_EINVAL;
  }
  if (num_tokens == 0 || batch_size == 0 || max_seqlen_q == 0) return REL_ATTN_OK;

  AttnParams& P = *P_out;
  P = AttnParams{};
  P.q = q;
  P.k = key_cache;
  P.v = value_cache;
  P.block_table = block_table;
  P.seqlens_k = cache_seqlens;
  P.cu_q = cu_seqlens_q;
  P.rel = rel_logits;
  P.out = out;
  P.ws_o = num_splits > 1 ? reinterpret_cast<float*>(workspace) : nullptr;
  P.ws_lse = num_splits > 1 ? P.ws_o + (size_t)num_splits * num_tokens * num_heads * head_dim : nullptr;
  P.T = num_tokens;
  P.B = batch_size;
  P.max_q = max_seqlen_q;
  P.max_blocks = max_blocks_per_seq;
  P.H = num_heads;
  P.Hkv = num_kv_heads;
  P.G = G;
  P.num_blocks = num_blocks;
  P.bs = block_size;
  P.E = rel_extent;
  P.scale_log2 = softmax_scale * kLog2e;
  P.causal = causal;
  P.wl = window_left;
  P.wr = window_right;
  P.splits = num_splits;

  {
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    P.kv_cap = cap > 0x7fffffff ? 0x7fffffff : (int)cap;
  }
  P.bs_log2 = -1;
  for (int k = 0; k < 31; ++k)
    if ((1 << k) == block_size) P.bs_log2 = k;
  // Keys per split of the decode kernel: the longest key range a request can
  // have (its page-table capacity, or the window span) cut into num_splits
  // pieces of whole 16-key tiles.
  {
    int64_t span = (int64_t)max_blocks_per_seq * block_size;
    if (window_left >= 0) {
      const int64_t right = window_right >= 0 ? window_right : (causal ? 0 : span);
      const int64_t w = (int64_t)window_left + right + max_seqlen_q + 16;
      if (w < span) span = w;
    }
    int64_t chunk = (span + num_splits - 1) / num_splits;
    chunk = (chunk + 15) / 16 * 16;
    if (chunk < 16) chunk = 16;
    P.dec_chunk = chunk > (1 << 30) ? (1 << 30) : (int)chunk;
  }
  *launch = true;
  return REL_ATTN_OK;
}

// The attention kernels of one call: partials into the workspace when the
// call splits, else the final output.
int launch_attention(AttnParams& P, int dtype, int head_dim, hipStream_t s) {
  const int bf16 = dtype == REL_ATTN_BF16;
  if (relattn::decode_supported(P, bf16, head_dim)) {
    if (relattn::launch_decode(P, head_dim, s) != 0) return REL_ATTN_ELAUNCH;
    // requests with more than 16 packed rows go to the prefill kernel
    P.mode = 1;
    if ((int64_t)P.max_q * P.G > relattn::kDecodeMaxRows) {
      const int rc = relattn::prefill_supported(P, bf16, head_dim) ? relattn::launch_prefill(P, s)
                                                                   : relattn::launch_general(P, bf16, head_dim, s);
      if (rc != 0) return REL_ATTN_ELAUNCH;
    }
  } else {
    P.mode = 0;
    if (relattn::launch_general(P, bf16, head_dim, s) != 0) return REL_ATTN_ELAUNCH;
  }
  return REL_ATTN_OK;
}

}  // namespace

#define REL_ATTN_ARGS                                                                                    \
  q, key_cache, value_cache, block_table, cache_seqlens, cu_seqlens_q, rel_logits, out, dtype,         \
      num_tokens, batch_size, max_seqlen_q, max_blocks_per_seq, num_heads, num_kv_heads, head_dim,     \
      num_blocks, block_size, rel_extent, softmax_scale, causal, window_left, window_right, num_splits, \
      workspace, workspace_bytes, workspace_needed

extern "C" int rel_attn_fwd(const void* q, const void* key_cache, const void* value_cache,
                            const int32_t* block_table, const int32_t* cache_seqlens,
                            const int32_t* cu_seqlens_q, const void* rel_logits, void* out, int dtype,
                            int num_tokens, int batch_size, int max_seqlen_q, int max_blocks_per_seq,
                            int num_heads, int num_kv_heads, int head_dim, int num_blocks, int block_size,
                            int rel_extent, float softmax_scale, int causal, int window_left,
                            int window_right, int num_splits, void* workspace, size_t workspace_bytes,
                            size_t* workspace_needed, void* stream) {
  AttnParams P;
  bool launch = false;
  int rc = prepare(REL_ATTN_ARGS, &P, &launch);
  if (rc != REL_ATTN_OK || !launch) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  rc = launch_attention(P, dtype, head_dim, s);
  if (rc != REL_ATTN_OK) return rc;
  if (num_splits > 1 && relattn::launch_combine(P, dtype == REL_ATTN_BF16, head_dim, s) != 0)
    return REL_ATTN_ELAUNCH;
  return REL_ATTN_OK;
}

extern "C" int rel_attn_fwd_splits(const void* q, const void* key_cache, const void* value_cache,
                                   const int32_t* block_table, const int32_t* cache_seqlens,
                                   const int32_t* cu_seqlens_q, const void* rel_logits, void* out,
                                   int dtype, int num_tokens, int batch_size, int max_seqlen_q,
                                   int max_blocks_per_seq, int num_heads, int num_kv_heads, int head_dim,
                                   int num_blocks, int block_size, int rel_extent, float softmax_scale,
                                   int causal, int window_left, int window_right, int num_splits,
                                   void* workspace, size_t workspace_bytes, size_t* workspace_needed,
                                   void* stream) {
  AttnParams P;
  bool launch = false;
  int rc = prepare(REL_ATTN_ARGS, &P, &launch);
  if (rc != REL_ATTN_OK || !launch) return rc;
  return launch_attention(P, dtype, head_dim, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int rel_attn_fwd_lse(const void* q, const void* key_cache, const void* value_cache,
                                const int32_t* block_table, const int32_t* cache_seqlens,
                                const int32_t* cu_seqlens_q, const void* rel_logits, void* out, float* lse,
                                int dtype, int num_tokens, int batch_size, int max_seqlen_q,
                                int max_blocks_per_seq, int num_heads, int num_kv_heads, int head_dim,
                                int num_blocks, int block_size, int rel_extent, float softmax_scale,
                                int causal, int window_left, int window_right, int num_splits,
                                void* workspace, size_t workspace_bytes, size_t* workspace_needed,
                                void* stream) {
  // the log-sum-exps come out of the split merge: one split runs as two
  if (num_splits == 1) num_splits = 2;
  AttnParams P;
  bool launch = false;
  int rc = prepare(REL_ATTN_ARGS, &P, &launch);
  if (rc != REL_ATTN_OK || !launch) return rc;  // error, empty call or workspace query
  if (lse == nullptr) return REL_ATTN_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  rc = launch_attention(P, dtype, head_dim, s);
  if (rc != REL_ATTN_OK) return rc;
  P.lse_out = lse;
  if (relattn::launch_combine(P, dtype == REL_ATTN_BF16, head_dim, s) != 0) return REL_ATTN_ELAUNCH;
  return REL_ATTN_OK;
}

#undef REL_ATTN_ARGS

// ---- rel_attn_fwd_noalloc: the split-KV workspace in a static device array ----

// The scratch memory of rel_attn_fwd_noalloc: room for the fp32 split-KV
// workspace of calls that cannot allocate. Every GPU the library runs on
// holds its own copy until the process ends. In host code this name stands
// for no device address: kernels get the address hipGetSymbolAddress
// returns for the current device (scratch_address below).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device

// The device address of this GPU's scratch array. The stream must belong to
// the current device; the address is looked up once per device, with that
// device current, and kept.
int scratch_address(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return REL_ATTN_ELAUNCH;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return REL_ATTN_ELAUNCH;
    if (sdev != dev) return REL_ATTN_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return REL_ATTN_ELAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return REL_ATTN_OK;
}

}  // namespace

extern "C" size_t rel_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int rel_attn_fwd_noalloc(const void* q, const void* key_cache, const void* value_cache,
                                    const int32_t* block_table, const int32_t* cache_seqlens,
                                    const int32_t* cu_seqlens_q, const void* rel_logits, void* out,
                                    int dtype, int num_tokens, int batch_size, int max_seqlen_q,
                                    int max_blocks_per_seq, int num_heads, int num_kv_heads,
                                    int head_dim, int num_blocks, int block_size, int rel_extent,
                                    float softmax_scale, int causal, int window_left, int window_right,
                                    int num_splits, void* stream) {
  // every argument check, then the size check (a workspace of
  // kScratchBytes), run before anything touches a device: the placeholder
  // address only stands in for the scratch array in those checks and is
  // never used
  const size_t need = rel_attn_workspace_bytes(num_splits, num_tokens, num_heads, head_dim);
  void* workspace = nullptr;
  {
    AttnParams P;
    bool launch = false;
    void* const placeholder = reinterpret_cast<void*>(uintptr_t(256));
    const int rc = prepare(q, key_cache, value_cache, block_table, cache_seqlens, cu_seqlens_q, rel_logits, out,
                           dtype, num_tokens, batch_size, max_seqlen_q, max_blocks_per_seq, num_heads, num_kv_heads,
                           head_dim, num_blocks, block_size, rel_extent, softmax_scale, causal, window_left,
                           window_right, num_splits, placeholder, kScratchBytes, nullptr, &P, &launch);
    if (rc != REL_ATTN_OK || !launch) return rc;
  }
  if (need > 0) {
    const int rc = scratch_address(reinterpret_cast<hipStream_t>(stream), &workspace);
    if (rc != REL_ATTN_OK) return rc;
  }
  return rel_attn_fwd(q, key_cache, value_cache, block_table, cache_seqlens, cu_seqlens_q, rel_logits, out, dtype,
                      num_tokens, batch_size, max_seqlen_q, max_blocks_per_seq, num_heads, num_kv_heads, head_dim,
                      num_blocks, block_size, rel_extent, softmax_scale, causal, window_left, window_right,
                      num_splits, workspace, workspace ? kScratchBytes : 0, nullptr, stream);
}

extern "C" int rel_attn_combine(const void* workspace, size_t workspace_bytes, void* out, int dtype,
                                int num_tokens, int num_heads, int head_dim, int num_splits,
                                void* stream) {
  if (num_tokens < 0 || num_heads < 1 || num_splits < 2 || num_splits > kMaxSplits)
    return REL_ATTN_EINVAL;
  if (dtype != REL_ATTN_FP32 && dtype != REL_ATTN_BF16) return REL_ATTN_EUNSUPPORTED;
  if (!supported_head_dim(head_dim)) return REL_ATTN_EUNSUPPORTED;
  const size_t need = rel_attn_workspace_bytes(num_splits, num_tokens, num_heads, head_dim);
  if (workspace == nullptr || workspace_bytes < need || need == SIZE_MAX) return REL_ATTN_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return REL_ATTN_EINVAL;
  if (num_tokens == 0) return REL_ATTN_OK;
  if (out == nullptr) return REL_ATTN_EINVAL;
  AttnParams P{};
  P.out = out;
  P.ws_o = reinterpret_cast<float*>(const_cast<void*>(workspace));
  P.ws_lse = P.ws_o + (size_t)num_splits * num_tokens * num_heads * head_dim;
  P.T = num_tokens;
  P.H = num_heads;
  P.splits = num_splits;
  return relattn::launch_combine(P, dtype == REL_ATTN_BF16, head_dim, reinterpret_cast<hipStream_t>(stream)) == 0
             ? REL_ATTN_OK
             : REL_ATTN_ELAUNCH;
}
