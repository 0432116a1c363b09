// Host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer
// (built by tests/test_sanitizers.py together with the library's sources):
//
//   masks  every host mask-builder call over a sweep of shapes, steps and
//          flags, with exact-size buffers (an overrun of the caller's arrays
//          is reported by ASan), the invariants of each mask checked, the
//          step-run builder, the validator on random malformed masks, and
//          the builders' argument errors;
//   abi    every argument check of the attention entry points, with
//          descriptors that point at no memory (all rejected before any
//          device work), the workspace-size calls, and, with no GPU, the
//          "no device" error.
//
// Prints "ok" and exits 0 on success; exits 1 at the first mismatch (a
// sanitizer report aborts with its own exit code).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "lvsa.h"

#define CHECK(cond, ...)                           \
  do {                                             \
    if (!(cond)) {                                 \
      std::fprintf(stderr, __VA_ARGS__);           \
      std::fprintf(stderr, " (line %d)\n", __LINE__); \
      return 1;                                    \
    }                                              \
  } while (0)

namespace {

int check_mask(int32_t T, int32_t C, int32_t W, int32_t step, int32_t flags) {
  int32_t nnz = -1;
  CHECK(lvsa_mask_nnz(T, C, W, &nnz) == LVSA_OK, "nnz %d %d %d: %s", T, C, W, lvsa_last_error());
  const int32_t c_eff = C < T ? C : T;
  CHECK(nnz == T * c_eff, "nnz %d", nnz);
  // exact sizes, on the heap, so that a write past either array is caught
  std::vector<int32_t> rp(T + 1), ci(nnz);
  lvsa_mask_info info;
  CHECK(lvsa_build_mask(T, C, W, step, flags, rp.data(), ci.data(), nnz, &info) == LVSA_OK, "build %d %d %d %d %d: %s",
        T, C, W, step, flags, lvsa_last_error());
  CHECK(info.c_eff == c_eff && info.nnz == nnz, "info");
  for (int32_t t = 0; t <= T; ++t) CHECK(rp[t] == t * c_eff, "row_ptr");
  for (int32_t t = 0; t < T; ++t) {
    bool self = false;
    for (int32_t e = rp[t]; e < rp[t + 1]; ++e) {
      CHECK(ci[e] >= 0 && ci[e] < T, "frame out of range");
      if (e > rp[t]) CHECK(ci[e] > ci[e - 1], "row not ascending");
      self |= ci[e] == t;
    }
    CHECK(self, "row %d misses its own frame", t);
  }
  CHECK(lvsa_validate_mask(T, rp.data(), ci.data(), nnz) == LVSA_OK, "validate: %s", lvsa_last_error());
  return 0;
}

int masks() {
  const int32_t shapes[][2] = {{2, 1}, {3, 1}, {4, 2}, {5, 2}, {8, 3}, {21, 9}, {33, 13}};
  for (int32_t T = 1; T <= 140; ++T)
    for (const auto &cw : shapes)
      for (int32_t flags = 0; flags < 4; ++flags)
        for (int32_t step = 0; step < (T < 20 ? 2 * T + 1 : 5); ++step)
          if (check_mask(T, cw[0], cw[1], step * 7 + (step > 3 ? 1000 : 0), flags)) return 1;
  if (check_mask(600, 21, 9, 123, LVSA_ROT_MOD_T)) return 1;

  // a run of steps in one exact-size buffer
  {
    const int32_t T = 65, C = 33, W = 13, n = 50;
    int32_t nnz = 0;
    CHECK(lvsa_mask_nnz(T, C, W, &nnz) == LVSA_OK, "nnz");
    std::vector<int32_t> rp(T + 1), ci((size_t)nnz * n), one(nnz), rp1(T + 1);
    std::vector<lvsa_mask_info> info(n);
    CHECK(lvsa_build_mask_steps(T, C, W, 0, n, LVSA_ROT_MOD_T, rp.data(), ci.data(), (int64_t)nnz * n, info.data()) ==
              LVSA_OK,
          "steps: %s", lvsa_last_error());
    for (int32_t s = 0; s < n; ++s) {
      CHECK(lvsa_build_mask(T, C, W, s, LVSA_ROT_MOD_T, rp1.data(), one.data(), nnz, nullptr) == LVSA_OK, "one");
      CHECK(std::memcmp(one.data(), ci.data() + (size_t)s * nnz, sizeof(int32_t) * nnz) == 0, "step %d differs", s);
    }
    CHECK(lvsa_build_mask_steps(T, C, W, 0, n, 0, rp.data(), ci.data(), (int64_t)nnz * n - 1, nullptr) ==
              LVSA_ERR_CAPACITY, "steps capacity");
    CHECK(lvsa_build_mask_steps(T, C, W, INT32_MAX, 2, 0, rp.data(), ci.data(), (int64_t)nnz * n, nullptr) ==
              LVSA_ERR_ARG, "steps overflow");
  }

  // builder argument errors
  {
    int32_t rp[9], ci[32], nnz;
    CHECK(lvsa_build_mask(0, 4, 2, 0, 0, rp, ci, 32, nullptr) == LVSA_ERR_ARG, "T=0");
    CHECK(lvsa_build_mask(8, 1, 1, 0, 0, rp, ci, 32, nullptr) == LVSA_ERR_ARG, "C=1");
    CHECK(lvsa_build_mask(8, 4, 4, 0, 0, rp, ci, 32, nullptr) == LVSA_ERR_ARG, "W=C");
    CHECK(lvsa_build_mask(8, 4, 2, -1, 0, rp, ci, 32, nullptr) == LVSA_ERR_ARG, "step<0");
    CHECK(lvsa_build_mask(8, 4, 2, 0, 9, rp, ci, 32, nullptr) == LVSA_ERR_ARG, "flags");
    CHECK(lvsa_build_mask(8, 4, 2, 0, 0, nullptr, ci, 32, nullptr) == LVSA_ERR_ARG, "null");
    CHECK(lvsa_build_mask(8, 4, 2, 0, 0, rp, ci, 31, nullptr) == LVSA_ERR_CAPACITY, "cap");
    CHECK(lvsa_mask_nnz(8, 4, 2, nullptr) == LVSA_ERR_ARG, "nnz null");
    CHECK(lvsa_mask_nnz(1 << 20, 1 << 20, 2, &nnz) == LVSA_ERR_ARG, "nnz overflow");
  }

  // the validator on random, mostly malformed masks: it must only ever
  // return OK or MASK, never read outside the arrays it was given
  std::mt19937 rng(12345);
  for (int it = 0; it < 20000; ++it) {
    const int32_t T = 1 + (int32_t)(rng() % 12);
    const int32_t nnz = (int32_t)(rng() % 40);
    std::vector<int32_t> rp(T + 1), ci(nnz > 0 ? nnz : 1);
    for (auto &x : rp) x = (int32_t)(rng() % (nnz + 3)) - 1;
    if (rng() % 2) {
      rp[0] = 0;
      for (int32_t t = 1; t <= T; ++t) rp[t] = rp[t - 1] + (int32_t)(rng() % 4);
      rp[T] = nnz;
    }
    for (auto &x : ci) x = (int32_t)(rng() % (T + 4)) - 2;
    const int rc = lvsa_validate_mask(T, rp.data(), ci.data(), nnz);
    CHECK(rc == LVSA_OK || rc == LVSA_ERR_MASK, "validate rc %d", rc);
  }
  CHECK(lvsa_validate_mask(4, nullptr, nullptr, 0) == LVSA_ERR_ARG, "validate null");
  return 0;
}

lvsa_tensor rec(uintptr_t data, int64_t B = 1, int64_t H = 2, int64_t N = 512, int64_t D = 64) {
  lvsa_tensor x;
  x.data = reinterpret_cast<void *>(data);
  x.B = B;
  x.H = H;
  x.N = N;
  x.D = D;
  x.stride_n = D;
  x.stride_h = N * D;
  x.stride_b = H * N * D;
  x.dtype = LVSA_DTYPE_BF16;
  return x;
}

int abi(bool no_device) {
  const uintptr_t base = uintptr_t{1} << 32, sz = 2 * 512 * 64 * 2;
  lvsa_tensor q = rec(base), k = rec(base + sz), v = rec(base + 2 * sz), o = rec(base + 3 * sz);
  const int32_t *rp = reinterpret_cast<const int32_t *>(0x1000), *ci = reinterpret_cast<const int32_t *>(0x2000);
  auto attn = [&](const lvsa_tensor &a, const lvsa_tensor &b, const lvsa_tensor &c, lvsa_tensor d, int32_t T = 8,
                  int32_t nnz = 32, float scale = 0.f) { return lvsa_attention(&a, &b, &c, rp, ci, T, nnz, &d, scale, nullptr); };
  lvsa_tensor bad = q;
  bad.dtype = 0;
  CHECK(attn(bad, k, v, o) == LVSA_ERR_DTYPE, "dtype");
  bad = q;
  bad.D = 96;
  CHECK(attn(bad, k, v, o) == LVSA_ERR_SHAPE, "D");
  bad = q;
  bad.data = reinterpret_cast<void *>(base + 2);
  CHECK(attn(bad, k, v, o) == LVSA_ERR_SHAPE, "alignment");
  bad = q;
  bad.stride_n = 68;
  CHECK(attn(bad, k, v, o) == LVSA_ERR_SHAPE, "stride");
  CHECK(attn(q, rec(base + sz, 1, 2, 256), v, o) == LVSA_ERR_SHAPE, "shape mismatch");
  CHECK(attn(q, k, v, rec(base + sz / 2)) == LVSA_ERR_SHAPE, "out overlaps q");
  lvsa_tensor self = o;
  self.stride_h = 0;
  CHECK(attn(q, k, v, self) == LVSA_ERR_SHAPE, "self-overlapping out");
  CHECK(attn(q, k, v, o, 7) == LVSA_ERR_SHAPE, "N %% T");
  CHECK(attn(q, k, v, o, 0) == LVSA_ERR_ARG, "T = 0");
  CHECK(attn(q, k, v, o, 8, -1) == LVSA_ERR_ARG, "nnz < 0");
  CHECK(attn(q, k, v, o, 8, 32, 1.0f / 0.0f) == LVSA_ERR_ARG, "scale inf");
  CHECK(lvsa_attention(nullptr, &k, &v, rp, ci, 8, 32, &o, 0.f, nullptr) == LVSA_ERR_ARG, "null q");
  CHECK(lvsa_attention(&q, &k, &v, nullptr, ci, 8, 32, &o, 0.f, nullptr) == LVSA_ERR_ARG, "null row_ptr");

  int64_t bytes = 0;
  CHECK(lvsa_attention_workspace_bytes(1, 2, 512, 64, 8, &bytes) == LVSA_OK && bytes == 512, "ws bytes %lld",
        (long long)bytes);
  CHECK(lvsa_attention_workspace_bytes(1, 12, 121 * 1560, 128, 121, &bytes) == LVSA_OK && bytes > 0, "ws bytes");
  CHECK(lvsa_attention_workspace_bytes(0, 2, 512, 64, 8, &bytes) == LVSA_ERR_ARG, "ws B=0");
  CHECK(lvsa_attention_workspace_bytes(1, 2, 512, 64, 8, nullptr) == LVSA_ERR_ARG, "ws null");
  CHECK(lvsa_attention_workspace_bytes(1, 2, 513, 64, 8, &bytes) == LVSA_ERR_SHAPE, "ws N %% T");
  CHECK(lvsa_attention_workspace_bytes(int64_t{1} << 40, int64_t{1} << 40, 512, 64, 8, &bytes) == LVSA_ERR_ARG,
        "ws overflow");
  const uintptr_t ws = base + 8 * sz;
  auto attn_ws = [&](uintptr_t w, int64_t n) {
    return lvsa_attention_ws(&q, &k, &v, rp, ci, 8, 32, &o, 0.f, reinterpret_cast<void *>(w), n, nullptr);
  };
  CHECK(attn_ws(0, 512) == LVSA_ERR_ARG, "ws NULL");
  CHECK(attn_ws(ws + 8, 512) == LVSA_ERR_ARG, "ws alignment");
  CHECK(attn_ws(ws, 511) == LVSA_ERR_CAPACITY, "ws capacity");
  CHECK(attn_ws(base + 16, 512) == LVSA_ERR_ARG, "ws overlaps q");
  // the static-scratch entry point: argument errors and a key-norm table
  // too large for its scratch (stride-0 views), all before any device work
  CHECK(lvsa_attention_ws_static(&q, &k, &v, rp, ci, 0, 32, &o, 0.f, nullptr) == LVSA_ERR_ARG, "static T=0");
  CHECK(lvsa_attention_ws_static(&q, &k, &v, rp, ci, 7, 32, &o, 0.f, nullptr) == LVSA_ERR_SHAPE, "static N %% T");
  lvsa_tensor big = rec(base, 1, 4200, 1024);
  big.stride_h = 0;
  CHECK(lvsa_attention_ws_static(&big, &big, &big, rp, ci, 1024, 4096, &big, 0.f, nullptr) == LVSA_ERR_CAPACITY,
        "static capacity");
  if (no_device) {
    CHECK(attn(q, k, v, o) == LVSA_ERR_HIP, "no device");
    CHECK(attn_ws(ws, 512) == LVSA_ERR_HIP, "ws no device");
    CHECK(lvsa_attention_ws_static(&q, &k, &v, rp, ci, 8, 32, &o, 0.f, nullptr) == LVSA_ERR_HIP, "static no device");
    CHECK(std::strlen(lvsa_last_error()) > 0, "message");
  }
  return 0;
}

}  // namespace

int main(int argc, char **argv) {
  const char *what = argc > 1 ? argv[1] : "";
  int rc = 1;
  if (std::strcmp(what, "masks") == 0) rc = masks();
  if (std::strcmp(what, "abi") == 0) rc = abi(false);
  if (std::strcmp(what, "abi-no-device") == 0) rc = abi(true);
  if (rc == 0) std::printf("ok\n");
  return rc;
}
