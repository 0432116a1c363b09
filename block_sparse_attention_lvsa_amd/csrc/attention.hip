// Frame-block-sparse flash attention for gfx950 (CDNA4), bf16 in / bf16 out.
//
// What it computes: for every (b, h) and query token i of frame t, softmax
// attention of q_i over the key/value tokens of the frames listed for t in a
// CSR frame mask (gist.science explainer "LVSA: Training-Free Sparse
// Attention for Long Video Diffusion", Technical Summary §2: "Core
// Mechanism" restricts query frame t to A(t); "Complexity" gives the
// per-query cost O(C·P·d) -- the sparsity block is a whole frame of P
// tokens).
//
// Work decomposition.  One workgroup = one tile of BM query tokens of one
// frame t of one (b, h); NW wavefronts of 64 lanes each own 32 query rows.
// The workgroup walks its CSR row once, merging consecutive key frames into
// runs: tokens are frame-major, so a run of frames [f0, f1] is the one
// contiguous token range [f0·P, (f1+1)·P).  Each run is streamed in tiles of
// BN = 64 keys; only the last tile of a run is partial (P = 1560 is not a
// multiple of the MFMA tile, so that tail is masked).
//
// Per key tile, per wave (all on the matrix cores, bf16 -> fp32):
//   Sᵀ(32 keys × 32 queries) = K · Qᵀ    v_mfma_f32_32x32x16_bf16, K from LDS,
//                                         Q held in VGPRs for the whole tile.
//   In the 32x32 accumulator layout lane l holds query l%32 and keys
//   8i + 4(l/32) + j, so a query's row lives in lanes l and l^32: the row
//   max and sum are per-lane reductions plus one permlane32 swap.
//   Online softmax in the log2 domain with a lazily updated running max
//   (rescale only when the tile max exceeds it by more than 2^8, so exp2
//   arguments stay <= 8 and fp32 cannot overflow).
//   Oᵀ(d × 32 queries) += Vᵀ · Pᵀ         P (bf16) comes straight from the Sᵀ
//   accumulator registers; Vᵀ is staged transposed in LDS.
//
// K/V staging.  Global -> registers (16-byte loads, issued one tile ahead)
// -> LDS, double-buffered, one workgroup barrier per tile.  K rows are
// stored with a 16-byte pad (row pitch 272 B for d = 128) so the 16-byte
// MFMA-operand reads are conflict-free; V is written transposed (Vᵀ[d][key],
// pitch 136 B) so each lane's 8-key operand is two 8-byte reads.
//
// Launch order.  Workgroups are dispatched round-robin over the 8 XCDs; the
// block index is remapped so each XCD receives a contiguous range of
// (b, h, t, query-tile) work items: the query tiles of a frame and
// neighbouring frames (which share most of their key frames) run on the same
// XCD and hit in its L2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "lvsa_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

constexpr int kBN = 64;             // keys per LDS tile
constexpr int kNumXcd = 8;          // XCDs per MI355X
constexpr float kMaxLag = 8.0f;     // log2 slack of the lazily updated row max

struct Args {
  const u16 *q, *k, *v;
  u16 *o;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  const int32_t *row_ptr, *col_idx;
  int32_t nnz, T, P, H, q_tiles, n_wg;
  float scale_log2;  // softmax scale × log2(e)
};

// Walks one CSR row and yields maximal runs of consecutive frames as token
// ranges [ks, ke).  Every value is wave-uniform (scalar registers).
struct RunIter {
  const int32_t *cols;
  int32_t e, e_end, T, P;
  int32_t ks, ke;

  __device__ bool next_run() {
    while (e < e_end) {
      const int32_t f = cols[e++];
      if (f < 0 || f >= T) continue;  // malformed entry: skipped, never read
      int32_t f1 = f;
      while (e < e_end && f1 + 1 < T && cols[e] == f1 + 1) { ++f1; ++e; }
      ks = f * P;
      ke = (f1 + 1) * P;
      return true;
    }
    return false;
  }
};

__device__ __forceinline__ float swap_halves_max(float x) {
  // permlane32_swap(x, x) returns {x[l], x[l^32]} in some order per lane.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Packs the low (hi=false) or high (hi=true) bf16 halves of two words.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <int D, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;          // threads per workgroup
  static constexpr int BM = NW * 32;          // query rows per workgroup
  static constexpr int KP = D + 8;            // K tile row pitch (elements)
  static constexpr int VP = kBN + 4;          // Vᵀ tile row pitch (elements)
  static constexpr int K_ELEMS = kBN * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int CH = D / 8;            // 16-byte chunks per token row
  static constexpr int UNITS = (kBN / 4) * CH; // staging units: 4 keys × 1 chunk
  static constexpr int UPT = (UNITS + NT - 1) / NT;
  static constexpr int LDS_BYTES = 2 * (K_ELEMS + V_ELEMS) * 2;
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void lvsa_attn_fwd(Args a) {
  using C = Cfg<D, NW>;
  __shared__ __attribute__((aligned(16))) u16 lds[2 * (C::K_ELEMS + C::V_ELEMS)];
  u16 *const Ks0 = lds;
  u16 *const Vt0 = lds + 2 * C::K_ELEMS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;  // which half of the wave

  // ---- work item (XCD-contiguous remap of the dispatch order)
  int item;
  {
    const int bid = blockIdx.x, n = a.n_wg;
    const int x = bid % kNumXcd, j = bid / kNumXcd;
    const int per = n / kNumXcd, rem = n % kNumXcd;
    item = (x < rem) ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
  }
  const int qt = item % a.q_tiles;
  const int rest = item / a.q_tiles;
  const int t = rest % a.T;
  const int bh = rest / a.T;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int P = a.P;

  const u16 *kbase = a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const u16 *vbase = a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;

  // ---- Q fragment: 32 rows × D per wave, B-operand layout
  const int q_row = qt * C::BM + wave * 32 + l32;  // row within frame t
  const bool q_ok = q_row < P;
  const bool wave_live = (qt * C::BM + wave * 32) < P;  // wave-uniform
  bf16x8_t qf[D / 16];
  {
    const u16 *qp = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh +
                    ((int64_t)t * P + (q_ok ? q_row : 0)) * a.q_sn + hf * 8;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      bf16x8_t x = *reinterpret_cast<const bf16x8_t *>(qp + dc * 16);
      if (!q_ok) x = bf16x8_t{};
      qf[dc] = x;
    }
  }

  // ---- CSR row -> runs of key frames
  RunIter it;
  {
    int32_t rb = a.row_ptr[t], re = a.row_ptr[t + 1];
    rb = rb < 0 ? 0 : (rb > a.nnz ? a.nnz : rb);
    re = re < rb ? rb : (re > a.nnz ? a.nnz : re);
    it.cols = a.col_idx;
    it.e = rb;
    it.e_end = re;
    it.T = a.T;
    it.P = P;
    it.ks = it.ke = 0;
  }

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16_t{};
  float m_run = -INFINITY;  // running row max, log2 domain (lazy)
  float l_run = 0.f;        // this lane's partial row sum

  uint4 kreg[C::UPT][4], vreg[C::UPT][4];

  auto load_tile = [&](int pos, int kv) {
#pragma unroll
    for (int u = 0; u < C::UPT; ++u) {
      const int unit = tid + u * C::NT;
      const int kg = unit % (kBN / 4), c = unit / (kBN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kg * 4 + r;
        uint4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
        if (unit < C::UNITS && j < kv) {
          const int64_t tok = (int64_t)(pos + j);
          kx = *reinterpret_cast<const uint4 *>(kbase + tok * a.k_sn + c * 8);
          vx = *reinterpret_cast<const uint4 *>(vbase + tok * a.v_sn + c * 8);
        }
        kreg[u][r] = kx;
        vreg[u][r] = vx;
      }
    }
  };

  auto store_tile = [&](int buf) {
    u16 *Ks = Ks0 + buf * C::K_ELEMS;
    u16 *Vt = Vt0 + buf * C::V_ELEMS;
#pragma unroll
    for (int u = 0; u < C::UPT; ++u) {
      const int unit = tid + u * C::NT;
      if (unit >= C::UNITS) continue;
      const int kg = unit % (kBN / 4), c = unit / (kBN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<uint4 *>(Ks + (kg * 4 + r) * C::KP + c * 8) = kreg[u][r];
      // transpose 4 keys × 8 dims into 8 rows of Vᵀ, 4 keys (8 bytes) each
      const uint32_t w[4][4] = {
          {vreg[u][0].x, vreg[u][0].y, vreg[u][0].z, vreg[u][0].w},
          {vreg[u][1].x, vreg[u][1].y, vreg[u][1].z, vreg[u][1].w},
          {vreg[u][2].x, vreg[u][2].y, vreg[u][2].z, vreg[u][2].w},
          {vreg[u][3].x, vreg[u][3].y, vreg[u][3].z, vreg[u][3].w}};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        uint2 pk;
        if (e & 1) {
          pk.x = pack_hi(w[0][wi], w[1][wi]);
          pk.y = pack_hi(w[2][wi], w[3][wi]);
        } else {
          pk.x = pack_lo(w[0][wi], w[1][wi]);
          pk.y = pack_lo(w[2][wi], w[3][wi]);
        }
        *reinterpret_cast<uint2 *>(Vt + (c * 8 + e) * C::VP + kg * 4) = pk;
      }
    }
  };

  auto compute_tile = [&](int buf, int kv) {
    const u16 *Ks = Ks0 + buf * C::K_ELEMS;
    const u16 *Vt = Vt0 + buf * C::V_ELEMS;
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const u16 *kp = Ks + (kb * 32 + l32) * C::KP + hf * 8;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(kp + dc * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[dc], s[kb], 0, 0, 0);
      }
    }
    if (kv < kBN) {  // tail tile of a run: keys >= kv are not in A(t)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb * 32 + (e >> 2) * 8 + hf * 4 + (e & 3);
          if (key >= kv) s[kb][e] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    mx = swap_halves_max(mx);
    const float mt = mx * a.scale_log2;
    const bool need = mt > m_run + kMaxLag;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
      m_run = m_new;
    }
    const float neg_m = -m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], a.scale_log2, neg_m));
        s[kb][e] = p;
        l_run += p;
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[kb][m * 8 + e];
        const int key0 = kb * 32 + m * 16 + hf * 4;
#pragma unroll
        for (int dc = 0; dc < D / 32; ++dc) {
          const u16 *vp = Vt + (dc * 32 + l32) * C::VP + key0;
          const bf16x4_t lo = *reinterpret_cast<const bf16x4_t *>(vp);
          const bf16x4_t hi = *reinterpret_cast<const bf16x4_t *>(vp + 8);
          const bf16x8_t vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, oacc[dc], 0, 0, 0);
        }
      }
  };

  // ---- main loop over key tiles (double-buffered LDS, one barrier per tile)
  bool have = it.next_run();
  int pos = it.ks;
  int kv = have ? min(kBN, it.ke - pos) : 0;
  if (have) {
    load_tile(pos, kv);
    store_tile(0);
  }
  __syncthreads();
  int buf = 0;
  while (have) {
    // advance a copy of the iterator to the next tile
    int npos = pos + kBN, nkv = 0;
    bool has_next = true;
    if (npos >= it.ke) {
      has_next = it.next_run();
      npos = it.ks;
    }
    if (has_next) {
      nkv = min(kBN, it.ke - npos);
      load_tile(npos, nkv);
    }
    if (wave_live) compute_tile(buf, kv);
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    if (!has_next) break;
    buf ^= 1;
    pos = npos;
    kv = nkv;
  }

  // ---- epilogue: normalise, round to bf16, store
  if (!q_ok) return;
  const float l_tot = swap_halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  u16 *op = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + ((int64_t)t * P + q_row) * a.o_sn;
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4_t r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = (__bf16)(oacc[dc][i * 4 + j] * inv);
      *reinterpret_cast<bf16x4_t *>(op + dc * 32 + i * 8 + hf * 4) = r;
    }
}

// ------------------------------------------------------------------ host --

struct DeviceCheck {
  std::once_flag once[64];
  int ok[64] = {};
};
DeviceCheck g_dev;

int check_device(int *dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64)
    return lvsa::fail(LVSA_ERR_HIP, "no HIP device available (%s)", hipGetErrorString(e));
  std::call_once(g_dev.once[dev], [dev]() {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess && std::strncmp(p.gcnArchName, "gfx950", 6) == 0)
      g_dev.ok[dev] = 1;
  });
  if (!g_dev.ok[dev]) return lvsa::fail(LVSA_ERR_HIP, "device %d is not a gfx950 (MI355X) GPU", dev);
  *dev_out = dev;
  return LVSA_OK;
}

int check_tensor(const lvsa_tensor *x, const char *name) {
  if (!x || !x->data) return lvsa::fail(LVSA_ERR_ARG, "%s: NULL tensor or data pointer", name);
  if (x->dtype != LVSA_DTYPE_BF16) return lvsa::fail(LVSA_ERR_DTYPE, "%s: dtype %d, only bf16 is supported", name, x->dtype);
  if (x->B < 1 || x->H < 1 || x->N < 1) return lvsa::fail(LVSA_ERR_SHAPE, "%s: empty or negative B/H/N", name);
  if (x->D != 64 && x->D != 128) return lvsa::fail(LVSA_ERR_SHAPE, "%s: D=%lld, supported 64 and 128", name, (long long)x->D);
  if (reinterpret_cast<uintptr_t>(x->data) % 16) return lvsa::fail(LVSA_ERR_SHAPE, "%s: data not 16-byte aligned", name);
  if (x->stride_n < x->D || x->stride_b < 0 || x->stride_h < 0 || x->stride_n % 8 || x->stride_h % 8 || x->stride_b % 8)
    return lvsa::fail(LVSA_ERR_SHAPE, "%s: strides must be multiples of 8 elements with stride_n >= D", name);
  return LVSA_OK;
}

// Byte extent [lo, hi) touched by a tensor.
void extent(const lvsa_tensor *x, uintptr_t *lo, uintptr_t *hi) {
  const int64_t last = (x->B - 1) * x->stride_b + (x->H - 1) * x->stride_h + (x->N - 1) * x->stride_n + x->D;
  *lo = reinterpret_cast<uintptr_t>(x->data);
  *hi = *lo + (uintptr_t)last * 2;
}

bool overlaps(const lvsa_tensor *a, const lvsa_tensor *b) {
  uintptr_t a0, a1, b0, b1;
  extent(a, &a0, &a1);
  extent(b, &b0, &b1);
  return a0 < b1 && b0 < a1;
}

template <int D, int NW>
int launch(const Args &args, hipStream_t stream) {
  hipLaunchKernelGGL((lvsa_attn_fwd<D, NW>), dim3(args.n_wg), dim3(NW * 64), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return lvsa::fail(LVSA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return lvsa::ok();
}

}  // namespace

extern "C" int lvsa_attention(const lvsa_tensor *q, const lvsa_tensor *k, const lvsa_tensor *v,
                              const int32_t *row_ptr_dev, const int32_t *col_idx_dev,
                              int32_t T, int32_t nnz, lvsa_tensor *out, float scale,
                              void *stream) {
  int rc;
  if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k")) || (rc = check_tensor(v, "v")) ||
      (rc = check_tensor(out, "out")))
    return rc;
  for (const lvsa_tensor *x : {k, v, (const lvsa_tensor *)out})
    if (x->B != q->B || x->H != q->H || x->N != q->N || x->D != q->D)
      return lvsa::fail(LVSA_ERR_SHAPE, "q/k/v/out shapes differ");
  if (overlaps(out, q) || overlaps(out, k) || overlaps(out, v))
    return lvsa::fail(LVSA_ERR_SHAPE, "out overlaps an input tensor");
  if (T < 1) return lvsa::fail(LVSA_ERR_ARG, "T=%d: need T >= 1", T);
  if (q->N % T) return lvsa::fail(LVSA_ERR_SHAPE, "N=%lld is not a multiple of T=%d", (long long)q->N, T);
  if (q->N > INT32_MAX / 2) return lvsa::fail(LVSA_ERR_SHAPE, "N=%lld too large", (long long)q->N);
  if (!row_ptr_dev || !col_idx_dev || nnz < 0)
    return lvsa::fail(LVSA_ERR_ARG, "row_ptr/col_idx NULL or nnz < 0");
  if (!(scale == scale) || std::isinf(scale)) return lvsa::fail(LVSA_ERR_ARG, "scale is not finite");
  int dev;
  if ((rc = check_device(&dev))) return rc;

  const int D = (int)q->D;
  const int P = (int)(q->N / T);
  constexpr int NW = 4;
  const int BM = NW * 32;
  const int q_tiles = (P + BM - 1) / BM;
  const int64_t n_wg = (int64_t)q->B * q->H * T * q_tiles;
  if (n_wg > INT32_MAX) return lvsa::fail(LVSA_ERR_SHAPE, "grid of %lld workgroups too large", (long long)n_wg);

  Args a;
  a.q = static_cast<const u16 *>(q->data);
  a.k = static_cast<const u16 *>(k->data);
  a.v = static_cast<const u16 *>(v->data);
  a.o = static_cast<u16 *>(out->data);
  a.q_sb = q->stride_b; a.q_sh = q->stride_h; a.q_sn = q->stride_n;
  a.k_sb = k->stride_b; a.k_sh = k->stride_h; a.k_sn = k->stride_n;
  a.v_sb = v->stride_b; a.v_sh = v->stride_h; a.v_sn = v->stride_n;
  a.o_sb = out->stride_b; a.o_sh = out->stride_h; a.o_sn = out->stride_n;
  a.row_ptr = row_ptr_dev;
  a.col_idx = col_idx_dev;
  a.nnz = nnz;
  a.T = T;
  a.P = P;
  a.H = (int32_t)q->H;
  a.q_tiles = q_tiles;
  a.n_wg = (int32_t)n_wg;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) return launch<128, NW>(a, s);
  return launch<64, NW>(a, s);
}
