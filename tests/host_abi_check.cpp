// Host-only exercise of librelattn's C ABI argument checks, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code of the
// library (tests/test_host_sanitizers.py). Every call here returns before
// any device work: invalid arguments, workspace-size queries and empty
// calls. Device pointers are stand-in addresses that the host never
// dereferences. Exit status 0 when every return code is the expected one.
#include <climits>
#include <initializer_list>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "rel_attn.h"

static int g_fail = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

namespace {

void* const kDev = reinterpret_cast<void*>(uintptr_t(4096));  // never dereferenced

struct Args {
  const void* q = kDev;
  const void* k = kDev;
  const void* v = kDev;
  const int32_t* bt = static_cast<const int32_t*>(kDev);
  const int32_t* sl = static_cast<const int32_t*>(kDev);
  const int32_t* cu = static_cast<const int32_t*>(kDev);
  const void* rel = kDev;
  void* out = kDev;
  float* lse = static_cast<float*>(kDev);
  int dtype = REL_ATTN_BF16, T = 4, B = 2, maxq = 2, mb = 3, H = 8, Hkv = 2, D = 128, NB = 10, bs = 16, E = 4;
  float scale = 0.1f;
  int causal = 1, wl = -1, wr = -1, splits = 1;
  void* ws = nullptr;
  size_t wsb = 0;
  size_t* need = nullptr;
};

int fwd(const Args& a) {
  return rel_attn_fwd(a.q, a.k, a.v, a.bt, a.sl, a.cu, a.rel, a.out, a.dtype, a.T, a.B, a.maxq, a.mb, a.H, a.Hkv,
                      a.D, a.NB, a.bs, a.E, a.scale, a.causal, a.wl, a.wr, a.splits, a.ws, a.wsb, a.need, nullptr);
}
int fwd_splits(const Args& a) {
  return rel_attn_fwd_splits(a.q, a.k, a.v, a.bt, a.sl, a.cu, a.rel, a.out, a.dtype, a.T, a.B, a.maxq, a.mb, a.H,
                             a.Hkv, a.D, a.NB, a.bs, a.E, a.scale, a.causal, a.wl, a.wr, a.splits, a.ws, a.wsb,
                             a.need, nullptr);
}
int fwd_lse(const Args& a) {
  return rel_attn_fwd_lse(a.q, a.k, a.v, a.bt, a.sl, a.cu, a.rel, a.out, a.lse, a.dtype, a.T, a.B, a.maxq, a.mb,
                          a.H, a.Hkv, a.D, a.NB, a.bs, a.E, a.scale, a.causal, a.wl, a.wr, a.splits, a.ws, a.wsb,
                          a.need, nullptr);
}
int noalloc(const Args& a) {
  return rel_attn_fwd_noalloc(a.q, a.k, a.v, a.bt, a.sl, a.cu, a.rel, a.out, a.dtype, a.T, a.B, a.maxq, a.mb,
                              a.H, a.Hkv, a.D, a.NB, a.bs, a.E, a.scale, a.causal, a.wl, a.wr, a.splits, nullptr);
}

typedef int (*Entry)(const Args&);
const Entry kEntries[] = {fwd, fwd_splits, fwd_lse};

}  // namespace

int main() {
  // ---- return-code strings ----
  for (int c : {0, -1, -2, -3, -4, 1, -5, INT_MIN, INT_MAX}) {
    const char* s = rel_attn_strerror(c);
    CHECK(s != nullptr && std::strlen(s) > 0);
  }

  // ---- split counts: in [1, 512] or REL_ATTN_EINVAL, for any input ----
  const int vals[] = {INT_MIN, -1, 0, 1, 2, 3, 7, 16, 64, 100, 4096, 1 << 20, INT_MAX - 1, INT_MAX};
  for (int local : {0, 1})
    for (int b : vals)
      for (int q : vals)
        for (int hkv : {-1, 0, 1, 2, 4, 8, 65535, INT_MAX})
          for (int g : {1, 3, 16, 17})
            for (int kv : vals) {
              const long long hl = (long long)hkv * g;
              const int h = hl > INT_MAX ? INT_MAX : (hl < INT_MIN ? INT_MIN : (int)hl);
              const int r = rel_attn_num_splits(local, b, q, h, hkv, kv);
              CHECK(r == REL_ATTN_EINVAL || (r >= 1 && r <= 512));
            }

  // ---- workspace sizes ----
  CHECK(rel_attn_workspace_bytes(1, 100, 32, 128) == 0);
  CHECK(rel_attn_workspace_bytes(4, 64, 32, 128) == (size_t)4 * 64 * 32 * 129 * 4);
  CHECK(rel_attn_workspace_bytes(0, 64, 32, 128) == 0);
  CHECK(rel_attn_workspace_bytes(2, -1, 32, 128) == 0);
  CHECK(rel_attn_workspace_bytes(512, INT_MAX, INT_MAX, INT_MAX) == SIZE_MAX);
  CHECK(rel_attn_workspace_bytes(512, INT_MAX, 1 << 20, 128) == SIZE_MAX);
  CHECK(rel_attn_workspace_bytes(2, INT_MAX, 1, 128) == (size_t)2 * INT_MAX * 129 * 4);
  for (int s : vals)
    for (int t : vals)
      for (int h : vals)
        for (int d : {INT_MIN, -1, 0, 1, 64, 128, INT_MAX}) {
          const size_t n = rel_attn_workspace_bytes(s, t, h, d);
          if (s < 1 || t < 0 || h < 1 || d < 1 || s == 1) CHECK(n == 0);
        }

  // ---- invalid arguments: the same code from every entry point ----
  struct Bad {
    int code;
    void (*set)(Args&);
  };
  const Bad bad[] = {
      {REL_ATTN_EINVAL, [](Args& a) { a.H = 30; a.Hkv = 4; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.splits = 0; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.splits = 513; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.splits = INT_MIN; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.T = -1; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.B = INT_MIN; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.maxq = -5; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.mb = -1; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.bs = 0; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.NB = -1; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.E = -1; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.wl = -2; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.wr = INT_MIN; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.causal = 2; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.Hkv = 0; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.H = 0; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.scale = __builtin_nanf(""); }},
      {REL_ATTN_EINVAL, [](Args& a) { a.q = nullptr; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.out = nullptr; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.bt = nullptr; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.sl = nullptr; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.cu = nullptr; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.k = nullptr; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.rel = nullptr; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.NB = 0; }},
      {REL_ATTN_EUNSUPPORTED, [](Args& a) { a.dtype = 2; }},
      {REL_ATTN_EUNSUPPORTED, [](Args& a) { a.D = 96; }},
      {REL_ATTN_EUNSUPPORTED, [](Args& a) { a.D = INT_MAX; }},
      {REL_ATTN_EUNSUPPORTED, [](Args& a) { a.H = 64; a.Hkv = 2; }},
      {REL_ATTN_EUNSUPPORTED, [](Args& a) { a.B = 65536; }},
      {REL_ATTN_EWORKSPACE, [](Args& a) { a.splits = 4; }},
      {REL_ATTN_EWORKSPACE, [](Args& a) { a.splits = 4; a.ws = kDev; a.wsb = 100; }},
      {REL_ATTN_EINVAL, [](Args& a) { a.splits = 4; a.ws = reinterpret_cast<void*>(uintptr_t(4097)); a.wsb = 1 << 30; }},
      // a size past size_t: no workspace is accepted, whatever size it claims
      {REL_ATTN_EWORKSPACE, [](Args& a) { a.splits = 512; a.T = INT_MAX; a.H = 1 << 19; a.Hkv = 1 << 15; a.ws = kDev; a.wsb = SIZE_MAX; }},
  };
  for (size_t ei = 0; ei < sizeof(kEntries) / sizeof(kEntries[0]); ++ei)
    for (size_t bi = 0; bi < sizeof(bad) / sizeof(bad[0]); ++bi) {
      Args a;
      bad[bi].set(a);
      const int got = kEntries[ei](a);
      if (got != bad[bi].code) std::fprintf(stderr, "entry %zu, case %zu: got %d\n", ei, bi, got);
      CHECK(got == bad[bi].code);
    }
  {
    Args a;  // NULL lse in a call that would launch
    a.splits = 4;
    a.ws = kDev;
    a.wsb = size_t(1) << 30;
    a.lse = nullptr;
    CHECK(fwd_lse(a) == REL_ATTN_EINVAL);
  }

  // ---- workspace queries and empty calls return before any device work ----
  for (Entry e : kEntries) {
    for (int s : {1, 2, 8, 512})
      for (int t : {0, 1, 4, 1000, INT_MAX})
        for (int h : {8, 16, 1 << 20}) {
          Args a;
          size_t need = 12345;
          a.splits = s;
          a.T = t;
          a.H = h;
          a.Hkv = h / 8;
          a.need = &need;
          CHECK(e(a) == REL_ATTN_OK);
          const int s_eff = (e == fwd_lse && s == 1) ? 2 : s;
          CHECK(need == rel_attn_workspace_bytes(s_eff, t, h, 128));
        }
    Args a;
    a.T = 0;
    a.B = 0;
    a.q = nullptr;
    a.out = nullptr;
    CHECK(e(a) == REL_ATTN_OK);
    Args b;
    b.maxq = 0;  // no query rows anywhere
    b.ws = kDev;
    b.wsb = size_t(1) << 30;
    CHECK(e(b) == REL_ATTN_OK);
  }

  // ---- combine ----
  const size_t ws4 = rel_attn_workspace_bytes(4, 4, 8, 128);
  CHECK(rel_attn_combine(kDev, size_t(1) << 30, kDev, REL_ATTN_BF16, 4, 8, 128, 1, nullptr) == REL_ATTN_EINVAL);
  CHECK(rel_attn_combine(kDev, size_t(1) << 30, kDev, REL_ATTN_BF16, 4, 8, 128, 513, nullptr) == REL_ATTN_EINVAL);
  CHECK(rel_attn_combine(kDev, size_t(1) << 30, kDev, REL_ATTN_BF16, -1, 8, 128, 4, nullptr) == REL_ATTN_EINVAL);
  CHECK(rel_attn_combine(kDev, size_t(1) << 30, nullptr, REL_ATTN_BF16, 4, 8, 128, 4, nullptr) == REL_ATTN_EINVAL);
  CHECK(rel_attn_combine(kDev, size_t(1) << 30, kDev, 7, 4, 8, 128, 4, nullptr) == REL_ATTN_EUNSUPPORTED);
  CHECK(rel_attn_combine(kDev, size_t(1) << 30, kDev, REL_ATTN_BF16, 4, 8, 80, 4, nullptr) == REL_ATTN_EUNSUPPORTED);
  CHECK(rel_attn_combine(nullptr, size_t(1) << 30, kDev, REL_ATTN_BF16, 4, 8, 128, 4, nullptr) == REL_ATTN_EWORKSPACE);
  CHECK(rel_attn_combine(kDev, ws4 - 1, kDev, REL_ATTN_BF16, 4, 8, 128, 4, nullptr) == REL_ATTN_EWORKSPACE);
  CHECK(rel_attn_combine(kDev, SIZE_MAX, kDev, REL_ATTN_BF16, INT_MAX, 1 << 20, 128, 512, nullptr) ==
        REL_ATTN_EWORKSPACE);
  CHECK(rel_attn_combine(kDev, size_t(1) << 30, kDev, REL_ATTN_BF16, 0, 8, 128, 4, nullptr) == REL_ATTN_OK);

  // ---- the allocation-free entry point ----
  CHECK(rel_attn_noalloc_scratch_bytes() == size_t(32) << 20);
  for (size_t bi = 0; bi < sizeof(bad) / sizeof(bad[0]); ++bi) {
    if (bad[bi].code == REL_ATTN_EWORKSPACE) continue;  // it has no workspace argument
    Args a;
    a.splits = 4;
    bad[bi].set(a);
    if (a.ws != nullptr) continue;  // a workspace pointer case
    const int got = noalloc(a);
    if (got != bad[bi].code) std::fprintf(stderr, "noalloc, case %zu: got %d\n", bi, got);
    CHECK(got == bad[bi].code);
  }
  {
    Args a;  // needs more than the scratch array
    a.splits = 2;
    a.T = 8192;
    a.H = 8;
    CHECK(noalloc(a) == REL_ATTN_EWORKSPACE);
    a.splits = 512;  // a size past size_t
    a.T = INT_MAX;
    a.H = 1 << 19;
    a.Hkv = 1 << 15;
    CHECK(noalloc(a) == REL_ATTN_EWORKSPACE);
    a.Hkv = 1 << 16;  // argument checks come first
    a.H = 1 << 20;
    CHECK(noalloc(a) == REL_ATTN_EUNSUPPORTED);
    Args e;  // empty call
    e.T = 0;
    e.B = 0;
    e.q = nullptr;
    e.out = nullptr;
    CHECK(noalloc(e) == REL_ATTN_OK);
  }

  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host ABI checks: all passed\n");
  return 0;
}
