// Host mask builder: per-step CSR key-frame lists of LVSA.
//
// Sources: gist.science explainer "LVSA: Training-Free Sparse Attention for
// Long Video Diffusion", Technical Summary §2 "Core Mechanism" (A(t) = G ∪
// W(t), rotating global anchors, window bounds extended over anchors so the
// budget holds); TechWalker article on LVSA, §二 (C = training horizon in
// latent frames, Tper ≈ T/(C−W), extension done on the CPU, ~1.4 µs per
// frame) and §三 (anchors rotate with the denoising step, constant count).
//
// Construction.  The anchors are an arithmetic progression modulo T.  The
// expanded window of frame t is the run of C − n_g non-anchor frames nearest
// to t (ties to the lower index).  Among the non-anchor frames listed in
// ascending order that set is always one contiguous stretch, so it is grown
// with two cursors, one step per frame taken, and merged with the sorted
// anchors: O(C) per row, O(T·C) per step, no allocation beyond two O(T)
// scratch vectors.
#include <algorithm>
#include <new>
#include <vector>

#include "lvsa_internal.h"

namespace {

int check_domain(int32_t T, int32_t C, int32_t W, int32_t step, int32_t flags) {
  if (T < 1) return lvsa::fail(LVSA_ERR_ARG, "T=%d: need T >= 1", T);
  if (C < 2) return lvsa::fail(LVSA_ERR_ARG, "C=%d: need C >= 2", C);
  if (W < 1 || W > C - 1) return lvsa::fail(LVSA_ERR_ARG, "W=%d: need 1 <= W <= C-1 (C=%d)", W, C);
  if (step < 0) return lvsa::fail(LVSA_ERR_ARG, "step=%d: need step >= 0", step);
  if (flags != LVSA_ROT_MOD_TPER && flags != LVSA_ROT_MOD_T && flags != LVSA_FIXED_GRID &&
      flags != LVSA_WINDOW_ONLY)
    return lvsa::fail(LVSA_ERR_ARG, "flags=%d: unknown rotation flag", flags);
  return LVSA_OK;
}

int64_t nnz_of(int32_t T, int32_t C) { return (int64_t)T * (int64_t)std::min(C, T); }

}  // namespace

extern "C" int lvsa_mask_nnz(int32_t T, int32_t C, int32_t W, int32_t *nnz_out) {
  if (!nnz_out) return lvsa::fail(LVSA_ERR_ARG, "nnz_out is NULL");
  int rc = check_domain(T, C, W, 0, LVSA_ROT_MOD_TPER);
  if (rc) return rc;
  int64_t n = nnz_of(T, C);
  if (n > INT32_MAX) return lvsa::fail(LVSA_ERR_ARG, "T*min(C,T) = %lld exceeds int32", (long long)n);
  *nnz_out = (int32_t)n;
  return lvsa::ok();
}

namespace {

int build_mask(int32_t T, int32_t C, int32_t W, int32_t step, int32_t flags, int32_t *row_ptr,
               int32_t *col_idx, int32_t cap, lvsa_mask_info *info) {
  int rc = check_domain(T, C, W, step, flags);
  if (rc) return rc;
  if (!row_ptr || !col_idx) return lvsa::fail(LVSA_ERR_ARG, "row_ptr/col_idx is NULL");
  const int64_t need = nnz_of(T, C);
  if (need > INT32_MAX) return lvsa::fail(LVSA_ERR_ARG, "mask of %lld entries exceeds int32", (long long)need);
  if (cap < need)
    return lvsa::fail(LVSA_ERR_CAPACITY, "col_idx capacity %d < required %lld", cap, (long long)need);

  const int32_t c_eff = std::min(C, T);
  lvsa_mask_info mi{c_eff, 0, 0, 0, (int32_t)need};

  if (T <= C) {  // dense: the budget covers the whole sequence
    for (int32_t t = 0; t <= T; ++t) row_ptr[t] = t * c_eff;
    for (int32_t t = 0; t < T; ++t)
      for (int32_t f = 0; f < T; ++f) col_idx[(int64_t)t * T + f] = f;
    if (info) *info = mi;
    return lvsa::ok();
  }

  // Anchor schedule: spacing, count, offset of this step (no anchors for the
  // window-only ablation).
  const bool anchored = flags != LVSA_WINDOW_ONLY;
  const int32_t t_per = anchored ? (T + (C - W) - 1) / (C - W) : 0;
  const int32_t n_g = anchored ? (T + t_per - 1) / t_per : 0;
  int32_t o = 0;
  if (flags == LVSA_ROT_MOD_TPER) o = step % t_per;
  else if (flags == LVSA_ROT_MOD_T) o = step % T;
  mi.t_per = t_per;
  mi.n_anchor = n_g;
  mi.offset = o;

  std::vector<uint8_t> is_anchor(T, 0);
  std::vector<int32_t> anchors;
  anchors.reserve(n_g);
  for (int32_t k = 0; k < n_g; ++k) {
    int32_t f = (int32_t)(((int64_t)o + (int64_t)k * t_per) % T);
    is_anchor[f] = 1;
  }
  std::vector<int32_t> free_frames;  // non-anchor frames, ascending
  free_frames.reserve(T - n_g);
  for (int32_t f = 0; f < T; ++f) {
    if (is_anchor[f]) anchors.push_back(f);
    else free_frames.push_back(f);
  }
  const int32_t budget = C - n_g;          // window frames per query frame
  const int32_t n_free = (int32_t)free_frames.size();

  // first_free_at[t] = index in free_frames of the first non-anchor >= t.
  int32_t cursor = 0;
  int32_t *out = col_idx;
  for (int32_t t = 0; t < T; ++t) {
    while (cursor < n_free && free_frames[cursor] < t) ++cursor;
    // Stretch [lo, hi) of free_frames, grown nearest-first around t.
    int32_t lo = cursor, hi = cursor;
    for (int32_t taken = 0; taken < budget; ++taken) {
      const bool has_l = lo > 0, has_r = hi < n_free;
      if (has_l && (!has_r || (t - free_frames[lo - 1]) <= (free_frames[hi] - t))) --lo;
      else ++hi;
    }
    // Merge the sorted anchors with the sorted stretch.
    int32_t a = 0, w = lo;
    while (a < n_g || w < hi) {
      if (w >= hi || (a < n_g && anchors[a] < free_frames[w])) *out++ = anchors[a++];
      else *out++ = free_frames[w++];
    }
    row_ptr[t] = t * c_eff;
  }
  row_ptr[T] = T * c_eff;
  if (info) *info = mi;
  return lvsa::ok();
}

int build_mask_steps(int32_t T, int32_t C, int32_t W, int32_t step0, int32_t n_steps, int32_t flags,
                     int32_t *row_ptr, int32_t *col_idx, int64_t cap, lvsa_mask_info *info) {
  if (n_steps < 1) return lvsa::fail(LVSA_ERR_ARG, "n_steps=%d: need n_steps >= 1", n_steps);
  int rc = check_domain(T, C, W, step0, flags);
  if (rc) return rc;
  if ((int64_t)step0 + n_steps - 1 > INT32_MAX)
    return lvsa::fail(LVSA_ERR_ARG, "step0 + n_steps - 1 exceeds int32");
  if (!row_ptr || !col_idx) return lvsa::fail(LVSA_ERR_ARG, "row_ptr/col_idx is NULL");
  const int64_t nnz = nnz_of(T, C);
  if (nnz > INT32_MAX) return lvsa::fail(LVSA_ERR_ARG, "mask of %lld entries exceeds int32", (long long)nnz);
  if (cap < nnz * n_steps)
    return lvsa::fail(LVSA_ERR_CAPACITY, "col_idx capacity %lld < required %lld", (long long)cap,
                      (long long)(nnz * n_steps));
  // Every step's row offsets are the same (t * c_eff), so the first call
  // writes row_ptr and the others only their own block of col_idx.
  std::vector<int32_t> scratch_rp(T + 1);
  for (int32_t i = 0; i < n_steps; ++i) {
    rc = build_mask(T, C, W, step0 + i, flags, i == 0 ? row_ptr : scratch_rp.data(),
                    col_idx + (int64_t)i * nnz, (int32_t)nnz, info ? info + i : nullptr);
    if (rc) return rc;
  }
  return lvsa::ok();
}

}  // namespace

// The C entry points: no C++ exception crosses the boundary (host memory
// exhaustion in the builders' scratch vectors becomes an error status).
extern "C" int lvsa_build_mask(int32_t T, int32_t C, int32_t W, int32_t step, int32_t flags,
                               int32_t *row_ptr, int32_t *col_idx, int32_t cap,
                               lvsa_mask_info *info) {
  try {
    return build_mask(T, C, W, step, flags, row_ptr, col_idx, cap, info);
  } catch (const std::bad_alloc &) {
    return lvsa::fail(LVSA_ERR_ARG, "out of host memory building the mask (T=%d)", T);
  }
}

extern "C" int lvsa_build_mask_steps(int32_t T, int32_t C, int32_t W, int32_t step0, int32_t n_steps,
                                     int32_t flags, int32_t *row_ptr, int32_t *col_idx, int64_t cap,
                                     lvsa_mask_info *info) {
  try {
    return build_mask_steps(T, C, W, step0, n_steps, flags, row_ptr, col_idx, cap, info);
  } catch (const std::bad_alloc &) {
    return lvsa::fail(LVSA_ERR_ARG, "out of host memory building the masks (T=%d)", T);
  }
}

extern "C" int lvsa_validate_mask(int32_t T, const int32_t *row_ptr, const int32_t *col_idx,
                                  int32_t nnz) {
  if (T < 1 || nnz < 0) return lvsa::fail(LVSA_ERR_ARG, "T=%d nnz=%d out of domain", T, nnz);
  if (!row_ptr || (!col_idx && nnz > 0)) return lvsa::fail(LVSA_ERR_ARG, "row_ptr/col_idx is NULL");
  if (row_ptr[0] != 0) return lvsa::fail(LVSA_ERR_MASK, "row_ptr[0]=%d, expected 0", row_ptr[0]);
  if (row_ptr[T] != nnz) return lvsa::fail(LVSA_ERR_MASK, "row_ptr[T]=%d, expected nnz=%d", row_ptr[T], nnz);
  for (int32_t t = 0; t < T; ++t) {
    const int32_t b = row_ptr[t], e = row_ptr[t + 1];
    if (e <= b) return lvsa::fail(LVSA_ERR_MASK, "row %d is empty or row_ptr decreases", t);
    if (b < 0 || e > nnz) return lvsa::fail(LVSA_ERR_MASK, "row %d offsets [%d,%d) outside [0,%d]", t, b, e, nnz);
    for (int32_t i = b; i < e; ++i) {
      const int32_t f = col_idx[i];
      if (f < 0 || f >= T) return lvsa::fail(LVSA_ERR_MASK, "row %d entry %d = %d outside [0,%d)", t, i - b, f, T);
      if (i > b && f <= col_idx[i - 1])
        return lvsa::fail(LVSA_ERR_MASK, "row %d not ascending/unique at entry %d", t, i - b);
    }
  }
  return lvsa::ok();
}
