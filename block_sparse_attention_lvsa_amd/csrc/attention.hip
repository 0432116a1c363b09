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
// Work decomposition.  One workgroup = one tile of BM = 32·NW query tokens
// of one frame t of one (b, h); each of its NW wavefronts owns 32 query
// rows.  The last tile of a frame is partial when BM does not divide P (Wan
// latents: P = 1560 = 12·128 + 24); its idle waves only join the loads and
// barriers, and the SIMDs they sit on run the other resident workgroups'
// waves meanwhile (packing the remainders of several frames into one tile
// measured slower: the merged iteration costs more than the idle waves).
//
// Key iteration.  The workgroup walks its CSR row once, merging consecutive
// key frames into runs: tokens are frame-major, so a run of frames [f0, f1]
// is the one contiguous token range [f0·P, (f1+1)·P).  Each run is streamed
// in tiles of BN keys; only the last tile of a run is partial, and its
// missing keys are masked.
//
// Per key tile, per wave (all on the matrix cores, bf16 -> fp32):
//   Sᵀ(32 keys × 32 queries) = K · Qᵀ    v_mfma_f32_32x32x16_bf16, K from LDS,
//                                         Q held in VGPRs for the whole loop.
//   In the 32x32 accumulator layout lane l holds query l%32 and keys
//   8i + 4(l/32) + j, so a query's row lives in lanes l and l^32: the row
//   max and sum are per-lane reductions plus one permlane32 swap.
//   Online softmax in the log2 domain with a lazily updated running max
//   (rescale only when the tile max exceeds it by more than 2^8, so exp2
//   arguments stay <= 8 and fp32 cannot overflow); or, given per-frame
//   key norms, a fixed per-row reference from a Cauchy-Schwarz bound,
//   subtracted by starting the Q·Kᵀ chain from it.
//   Oᵀ(d × 32 queries) += Vᵀ · Pᵀ         P (bf16) comes straight from the Sᵀ
//                                         accumulator registers; the Vᵀ
//                                         operand is built by transposing
//                                         LDS reads (ds_read_b64_tr_b16).
//
// K/V staging.  Each tile's K and V rows go from global memory straight into
// LDS (buffer loads with the LDS-destination bit, 16 bytes per lane), double
// buffered: the loads of tile j+1 run while tile j is computed, one
// workgroup barrier per tile.  16-byte chunks are XOR-swizzled by key so
// every MFMA operand read is bank-conflict free.
//
// Launch order.  Workgroups are dispatched round-robin over the 8 XCDs; each
// XCD receives a contiguous range of (b, h, t, query-tile) work items: the
// query tiles of a frame and neighbouring frames (which share most of their
// key frames) run on the same XCD and hit in its L2.  With a workspace the
// items are taken from per-XCD counters, so XCDs that clock faster take over
// work from slower ones (see the work-item block in the kernel).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <utility>

#include "lvsa_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

// Tuning knobs (compile-time): waves per workgroup, the register budget
// expressed as resident waves per SIMD, keys per tile, and how many K operand
// reads run ahead of the Q·Kᵀ MFMA chain.
#ifndef LVSA_NW
#define LVSA_NW 4
#endif
#ifndef LVSA_WAVES_PER_SIMD
#define LVSA_WAVES_PER_SIMD 3
#endif
#ifndef LVSA_BN
#define LVSA_BN 32
#endif
#ifndef LVSA_KAHEAD
#define LVSA_KAHEAD 3
#endif

constexpr int kNumXcd = 8;          // XCDs per MI355X
constexpr float kMaxLag = 8.0f;     // log2 slack of the lazily updated row max
// Largest log2 gap a fixed softmax reference may leave below a row's true
// maximum: with the reference at most 96 above it (its bound, below), the
// largest probability of the row stays >= 2^-96, far inside the normal
// range of fp32 and bf16 (2^-126).
constexpr float kMaxRefGap = 96.0f;

struct Args {
  const u16 *q, *k, *v;
  u16 *o;
  int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int32_t q_sn, k_sn, v_sn, o_sn;  // token strides (elements; < 2^24)
  const int32_t *row_ptr, *col_idx;
  int32_t nnz, T, P, H, q_tiles, n_wg;
  float scale_log2;  // softmax scale × log2(e)
  // Per (b, h, frame), [B·H·T]: the largest key norm max_j |k_j|; or null:
  // then every wave uses the running-max softmax.
  const float *knorm;
  // Per-XCD work-item counters, zeroed before the launch, or null: then
  // workgroup i runs the (i mod 8)-th XCD's (i div 8)-th item.
  int *tickets;
  // With tickets: the last min(split_cap, range / 4) items of each XCD
  // range run as two halves of their CSR row, whose partial results (records
  // of kPartialFloats(D) floats per lane, slot x·split_cap + j) go to
  // `partial` and are merged by lvsa_combine; split_cap = 0 splits nothing.
  float *partial;
  int32_t split_cap;
};

// Read-only kernel inputs read at wave-uniform addresses go through the
// constant address space, so they become scalar loads served by the scalar
// cache instead of vector loads that each wait for memory.
typedef const __attribute__((address_space(4))) int32_t *const_i32p;
typedef const __attribute__((address_space(4))) float *const_f32p;

// Walks one CSR row and yields maximal runs of consecutive frames as token
// ranges [ks, ke).  Every value is wave-uniform (scalar registers).  An entry
// outside [0, T), or not above the last frame taken, is skipped, so a
// malformed row never causes an out-of-range read and never repeats a frame.
struct RunIter {
  const_i32p cols;
  int32_t e, e_end, T, P;
  int32_t last;  // last frame taken (-1 before the first)
  int32_t ks, ke;

  __device__ bool next_run() {
    while (e < e_end) {
      const int32_t f = cols[e++];
      if (f <= last || f >= T) continue;
      int32_t f1 = f;
      while (e < e_end && f1 + 1 < T && cols[e] == f1 + 1) { ++f1; ++e; }
      last = f1;
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

// LDS tile layout.  K and V tiles are kept in their natural [key][d] order
// (one 2·D-byte row per key), filled straight from global memory by
// global_load_lds (16 bytes per lane, 1 KB per wave instruction), with the
// 16-byte chunks of each row XOR-swizzled by key so that the MFMA operand
// reads are bank-conflict free:
//   K: chunk c of key j is stored at chunk c ^ (j mod CH)
//        -> the 16-byte Q·Kᵀ operand reads of 16 consecutive keys hit 16
//           different chunks.
//   V: chunk c of key j is stored at chunk c ^ (VSW·(j mod 4))
//        -> the transposing 8-byte reads that build the P·V operand (4
//           consecutive keys × 4 quads of d per 16-lane group) are spread
//           over distinct banks.
template <int D, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;          // threads per workgroup
  static constexpr int BM = NW * 32;          // query rows per workgroup (32 per wave)
  static constexpr int BN = LVSA_BN;          // keys per LDS tile
  static constexpr int KB = BN / 32;          // 32-key MFMA blocks per tile
  static constexpr int CH = D / 8;            // 16-byte chunks per key row
  static constexpr int ROWB = D * 2;          // bytes per key row
  static constexpr int TILE_BYTES = BN * ROWB;
  static constexpr int LOADS = TILE_BYTES / 1024;      // 1 KB wave loads per tile
  static constexpr int LOADS_PER_WAVE = LOADS / NW;
  static constexpr int VSW = CH / 4;          // V swizzle step
  static constexpr int KEYS_PER_LOAD = 64 / CH;       // keys per 1 KB wave load
  static constexpr int STAGES = 2;                    // LDS tile buffers (loads run one tile ahead)
  static constexpr int LDS_BYTES = STAGES * 2 * TILE_BYTES; // {K, V} × STAGES
  static_assert(LOADS % NW == 0, "tile loads must split evenly over the waves");
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;

// Word 3 of a raw buffer descriptor (CDNA: 32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

// The items are split into 8 contiguous ranges, one per XCD.
__device__ __forceinline__ void xcd_range(int n, int x, int *base, int *cnt) {
  const int per = n / kNumXcd, rem = n % kNumXcd;
  *base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  *cnt = per + (x < rem ? 1 : 0);
}

// Items of one XCD range run as two halves (the end of the range, where the
// last workgroups of a launch finish at different times; shorter items make
// that ragged end shorter).
__device__ __forceinline__ int split_count(int cap, int cnt) { return min(cap, cnt / 4); }

// Floats per lane in a partial record: the lane's O accumulators (D/2),
// its partial row sum, the row's reference, padding to 16 bytes.
__host__ __device__ constexpr int kPartialFloats(int d) { return d / 2 + 4; }

// One wave's state and steps.  Kept in a struct so that the per-tile step
// can be specialised on the LDS buffer (immediate LDS offsets).  A wave owns
// 32 query rows.
template <int D, int NW>
struct Block {
  using C = Cfg<D, NW>;

  char *lds;
  int lane, wave, l32, hf;
  float scale_log2;
  bf16x8_t qf[D / 16];         // the wave's Q rows, B-operand layout
  f32x16_t oacc[D / 32];       // Oᵀ accumulators (dims × 32 queries)
  float m_run;                 // running row max, log2 domain (lazily raised), or the fixed reference
  f32x16_t bias;               // with a fixed reference R: -R, the Q·Kᵀ chain's initial accumulator
  float l_run;                 // this lane's partial row sum
  int32_t kro[D / 16];         // LDS byte offsets of this lane's K operands
  int32_t vro[D / 32];         // LDS byte offsets of this lane's V source rows
  int32_t koffb[C::LOADS_PER_WAVE], voffb[C::LOADS_PER_WAVE];  // load byte offsets

  static constexpr int kTileOffK(int buf) { return buf * 2 * C::TILE_BYTES; }
  static constexpr int kTileOffV(int buf) { return buf * 2 * C::TILE_BYTES + C::TILE_BYTES; }

  __device__ __forceinline__ void init_offsets(int32_t k_sn, int32_t v_sn) {
    // Load i of this wave covers keys key0 + i·KEYS_PER_LOAD (one per group
    // of CH lanes); each lane writes stored chunk `pchunk` of its key's row,
    // which holds logical chunk pchunk ^ swizzle(key).
    const int key0 = wave * C::LOADS_PER_WAVE * C::KEYS_PER_LOAD + lane / C::CH;
    const int pchunk = lane % C::CH;
#pragma unroll
    for (int i = 0; i < C::LOADS_PER_WAVE; ++i) {
      const int key = key0 + i * C::KEYS_PER_LOAD;
      koffb[i] = (key * k_sn + (pchunk ^ (key & (C::CH - 1))) * 8) * 2;
      voffb[i] = (key * v_sn + (pchunk ^ (C::VSW * (key & 3))) * 8) * 2;
    }
    // K operand (Q·Kᵀ, A side): key kb·32 + l32, logical chunk 2·dc + hf.
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      kro[dc] = l32 * C::ROWB + (((dc * 2 + hf) ^ (l32 & (C::CH - 1))) * 16);
    // V operand (P·V, A side) by transposing 8-byte reads: in 16-lane group
    // g, source lane s points at key 4·hf + s/4 (+ 16m + 8e per MFMA) and at
    // dims 32·dc + 16·(g mod 2) + 4·(s mod 4) .. +3; the transpose then hands
    // each lane its own dim for 4 consecutive keys.
    const int s16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      const int c = dc * 4 + (g & 1) * 2 + ((s16 & 3) >> 1);
      vro[dc] = (4 * hf + (s16 >> 2)) * C::ROWB + ((c ^ (C::VSW * (s16 >> 2))) * 16) + (s16 & 1) * 8;
    }
  }

  // Starts the direct global->LDS load of the K (or V) rows [pos, pos+kv)
  // into LDS buffer `buf`.  The buffer descriptor ends at row pos+kv, so the
  // rows of a run's tail tile past its end are filled with zeros by the
  // hardware and nothing outside the run is read.
  template <bool IS_V>
  __device__ __forceinline__ void issue(int buf, const u16 *base, int32_t sn, int pos, int kv) {
    const u16 *tb = base + (int64_t)pos * sn;
    const int nrec = ((kv - 1) * sn + D) * 2;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)tb, 0, nrec, kBufferFlags);
    char *dst = lds + (IS_V ? kTileOffV(buf) : kTileOffK(buf)) + wave * C::LOADS_PER_WAVE * 1024;
#pragma unroll
    for (int i = 0; i < C::LOADS_PER_WAVE; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + i * 1024), 16, IS_V ? voffb[i] : koffb[i], 0, 0, 0);
  }

  // Sᵀ (keys × 32 queries) of the K tile in buffer KBUF.
  // With a fixed reference (FIXED) the chain starts from -R instead of 0, so
  // the accumulators come out as S·scale·log2e - R with no extra instruction
  // (the wave's Q rows are then pre-scaled by scale·log2e).
  template <int KBUF, bool FIXED>
  __device__ __forceinline__ void qk(f32x16_t (&sc)[C::KB]) const {
    const char *Kb = lds + kTileOffK(KBUF);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) sc[kb] = FIXED ? bias : f32x16_t{};
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const bf16x8_t kf = *(const lds_bf16x8 *)(Kb + kro[dc] + kb * 32 * C::ROWB);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[dc], sc[kb], 0, 0, 0);
      }
#if LVSA_KAHEAD
    // Issue order: LVSA_KAHEAD operand reads ahead of the dependent MFMA
    // chain, then one read per MFMA, so each MFMA finds its K operand
    // already loaded (the compiler's own order waits on every second read).
    __builtin_amdgcn_sched_group_barrier(0x100, LVSA_KAHEAD, 1);
#pragma unroll
    for (int i = 0; i < D / 16 * C::KB - LVSA_KAHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, LVSA_KAHEAD, 1);
#endif
  }

  // Masks the keys >= kv of a run's tail tile.
  __device__ __forceinline__ void mask_tail(f32x16_t (&sc)[C::KB], int kv) {
    if (kv < C::BN) {
      // Empty asm: keeps this wave-uniform branch a branch (no speculation
      // of the selects into every tile).
      asm volatile("" ::: "memory");
      // element e of block kb is key kb·32 + 8·(e/4) + 4·hf + e%4; compare
      // its lane-independent part against a per-lane threshold.
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const int thr = kv - kb * 32 - 4 * hf;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if ((e >> 2) * 8 + (e & 3) >= thr) sc[kb][e] = -INFINITY;
      }
    }
  }

  // Folds the tile's row maximum into m_run (raised lazily, only when it
  // would exceed it by more than 2^kMaxLag) and rescales O and the row sum
  // when it moves.
  __device__ __forceinline__ void fold_max(const f32x16_t (&sc)[C::KB]) {
    float mx = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
    mx = swap_halves_max(mx);
    const float mt = mx * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kMaxLag) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
      m_run = m_new;
    }
  }

  // Probabilities of a tile, rounded to bf16, in the MFMA B-operand order of
  // the P·V product: P = 2^(S·scale·log2e − m_run) once the tile's maximum
  // has been folded into m_run, or, with a fixed reference (FIXED), straight
  // from the accumulators, which already hold S·scale·log2e − R.  The row
  // sum takes the same rounded values, so the normalised weights sum to one.
  template <bool FIXED>
  __device__ __forceinline__ void probs(const f32x16_t (&sc)[C::KB], bf16x8_t (&pb)[2 * C::KB]) {
    const float neg_m = -m_run;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pb[kb * 2 + m][e] = (__bf16)__builtin_amdgcn_exp2f(
              FIXED ? sc[kb][m * 8 + e] : __builtin_fmaf(sc[kb][m * 8 + e], scale_log2, neg_m));
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2_t pr = {pb[kb * 2 + m][e], pb[kb * 2 + m][e + 1]};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
        }
      }
  }

  // Oᵀ += Vᵀ·Pᵀ with the V tile in buffer VBUF.
  template <int VBUF>
  __device__ __forceinline__ void pv(const bf16x8_t (&pb)[2 * C::KB]) {
    const char *Vb = lds + kTileOffV(VBUF);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int krow = (kb * 32 + m * 16) * C::ROWB;
#pragma unroll
        for (int dc = 0; dc < D / 32; ++dc) {
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(Vb + vro[dc] + krow));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(Vb + vro[dc] + krow + 8 * C::ROWB));
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kb * 2 + m], oacc[dc], 0, 0, 0);
        }
      }
  }

  // One key tile from LDS buffer BUF.
  template <int BUF, bool FIXED>
  __device__ __forceinline__ void tile(int kv) {
    f32x16_t sc[C::KB];
    bf16x8_t pb[2 * C::KB];
    qk<BUF, FIXED>(sc);
    mask_tail(sc, kv);
    if constexpr (!FIXED) fold_max(sc);
    probs<FIXED>(sc, pb);
    pv<BUF>(pb);
  }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(LVSA_WAVES_PER_SIMD, LVSA_WAVES_PER_SIMD)))
void lvsa_attn_fwd(Args a) {
  using C = Cfg<D, NW>;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];  // K0 V0 K1 V1

  Block<D, NW> blk;
  blk.lds = lds;
  const int tid = threadIdx.x;
  blk.lane = tid & 63;
  blk.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  blk.l32 = blk.lane & 31;
  blk.hf = blk.lane >> 5;
  blk.scale_log2 = a.scale_log2;

  // ---- work item.  The items are split into 8 contiguous ranges, one per
  // XCD, so that the query tiles of a frame and neighbouring frames (which
  // share most key frames) run on one XCD and share its L2.  Statically,
  // workgroup i runs the (i div 8)-th item of XCD i mod 8's range (the
  // dispatcher deals workgroups round-robin over the XCDs).  With ticket
  // counters, a workgroup takes the next item of the range of the XCD it
  // runs on, and once that range is used up, of the others: the XCDs of one
  // part run at different speeds (up to ~7% apart), and a static split
  // leaves the fast ones idle while the slowest finishes.  More workgroups
  // than items are launched; the ones that find no item left exit.
  int item, half = -1, slot = 0;
  if (a.tickets) {
    // The item (and, for a half, which half and its record slot) is
    // broadcast through the first words of LDS tile buffer 1: the first tile
    // loads (buffer 0) do not touch them, and every wave reads them before
    // the barrier that precedes the loads into buffer 1.  (A separate
    // __shared__ word measured 2.5-6% slower, from the code it changes: more
    // LDS alone, up to 48 KB per workgroup, costs nothing.)
    int *const s_item = reinterpret_cast<int *>(lds + 2 * C::TILE_BYTES);
    if (tid == 0) {
      unsigned xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      int got = -1, gh = -1, gs = 0;
      for (int d = 0; d < kNumXcd && got < 0; ++d) {
        const int x = (int)((xcc + d) % kNumXcd);
        int base, cnt;
        xcd_range(a.n_wg, x, &base, &cnt);
        // A range hands out cnt + S tickets: its first cnt - S items whole,
        // then each of its last S items as two halves.
        const int S = split_count(a.split_cap, cnt), whole = cnt - S;
        // system scope: performed past the per-XCD L2s, so every XCD sees
        // one counter
        const int k = __hip_atomic_fetch_add(a.tickets + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        if (k < whole) {
          got = base + k;
        } else if (k < cnt + S) {
          const int j = (k - whole) >> 1;
          got = base + whole + j;
          gh = (k - whole) & 1;
          gs = x * a.split_cap + j;
        }
      }
      s_item[0] = got;
      s_item[1] = gh;
      s_item[2] = gs;
    }
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(s_item[0]);
    half = __builtin_amdgcn_readfirstlane(s_item[1]);
    slot = __builtin_amdgcn_readfirstlane(s_item[2]);
    if (item < 0) return;  // every item is taken (uniform: all waves leave)
  } else {
    const int x = blockIdx.x % kNumXcd, j = blockIdx.x / kNumXcd;
    int base, cnt;
    xcd_range(a.n_wg, x, &base, &cnt);
    item = base + j;
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

  // ---- Q fragments: the wave's 32 rows × D, B-operand layout
  const int row0 = qt * C::BM + blk.wave * 32;  // first row of this wave within frame t
  {
    const int r = row0 + blk.l32;
    const bool ok = r < P;
    const u16 *qp = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh + ((int64_t)t * P + (ok ? r : 0)) * a.q_sn +
                    blk.hf * 8;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      bf16x8_t x = *reinterpret_cast<const bf16x8_t *>(qp + dc * 16);
      if (!ok) x = bf16x8_t{};
      blk.qf[dc] = x;
    }
  }
#pragma unroll
  for (int i = 0; i < D / 32; ++i) blk.oacc[i] = f32x16_t{};
  blk.m_run = -INFINITY;
  blk.l_run = 0.f;
  blk.init_offsets(a.k_sn, a.v_sn);
  // Whether the wave has rows inside the frame (the last query tile of a
  // frame may not fill every wave), as a scalar, so the per-tile test is a
  // scalar branch rather than a vector compare.
  const int compute = __builtin_amdgcn_readfirstlane(row0 < P ? 1 : 0);

  // ---- CSR row -> runs of key frames
  RunIter it;
  int32_t rb, re;  // the whole CSR row
  {
    const const_i32p rp = (const_i32p)a.row_ptr;
    rb = rp[t];
    re = rp[t + 1];
    rb = rb < 0 ? 0 : (rb > a.nnz ? a.nnz : rb);
    re = re < rb ? rb : (re > a.nnz ? a.nnz : re);
    it.cols = (const_i32p)a.col_idx;
    it.e = rb;
    it.e_end = re;
    it.T = a.T;
    it.P = P;
    it.last = -1;
    it.ks = it.ke = 0;
  }
  int n_tiles = 0;  // tiles of the whole row
  {
    RunIter c = it;
    while (c.next_run()) n_tiles += (c.ke - c.ks + C::BN - 1) / C::BN;
  }
  int n_walk = n_tiles;  // tiles this workgroup walks
  if (half >= 0) {
    // A half walks entries [rb, mid) or [mid, re) of the row, the second
    // starting from the walk's state at mid, so that together they keep
    // exactly the entries the whole walk keeps.
    const int32_t mid = rb + (re - rb) / 2;
    RunIter c = it;
    c.e_end = mid;
    int first = 0;
    while (c.next_run()) first += (c.ke - c.ks + C::BN - 1) / C::BN;
    if (half == 0) {
      it.e_end = mid;
      n_walk = first;
    } else {
      it.e = mid;
      it.last = c.last;
      n_walk = 0;
      RunIter d = it;
      while (d.next_run()) n_walk += (d.ke - d.ks + C::BN - 1) / C::BN;
    }
  }

  // ---- softmax reference.  Without a key-norm table: the running max,
  // raised lazily.  With one: by Cauchy-Schwarz every score of query i lies
  // within ±|q_i|·K, K the largest key norm over the row's frames, so
  // R_i = scale·log2e·|q_i|·K·(1 + 2^-8) bounds every exponent (the factor
  // covers the rounding of the fp32 norms and of the MFMA dot products).  A
  // wave whose lanes all have 2·R_i <= kMaxRefGap (the bound cannot sit more
  // than 2·R_i above a row's true maximum) takes R_i as a fixed reference:
  // no running max, no rescale, and the subtraction is folded into the
  // Q·Kᵀ chain's initial accumulator.  Other waves keep the running max.
  bool fixed = false;
  if (a.knorm) {
    const const_f32p fn = (const_f32p)(a.knorm + (int64_t)bh * a.T);
    float kn = 0.f;
    for (int32_t e = rb; e < re; ++e) {  // the whole row, so both halves decide alike
      const int32_t f = it.cols[e];
      if (f >= 0 && f < a.T) kn = fmaxf(kn, fn[f]);
    }
    float ss = 0.f;  // |q'_i|^2 of the scaled, rounded rows
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)(__bf16)((float)blk.qf[dc][e] * a.scale_log2);
        ss = __builtin_fmaf(x, x, ss);
      }
    ss = swap_halves_sum(ss);  // each lane half holds half of the row
    const float r_ref = __builtin_sqrtf(ss) * kn * (1.0f + 1.0f / 256.0f);
    fixed = __builtin_amdgcn_ballot_w64(!(2.0f * r_ref <= kMaxRefGap)) == 0;
    if (fixed) {
      blk.m_run = r_ref;
#pragma unroll
      for (int e = 0; e < 16; ++e) blk.bias[e] = -r_ref;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
#pragma unroll
        for (int e = 0; e < 8; ++e) blk.qf[dc][e] = (__bf16)((float)blk.qf[dc][e] * a.scale_log2);
    }
  }

  // ---- main loop over key tiles: K and V double-buffered in LDS (tile j in
  // buffer j mod 2); the loads of tile j+1 run while tile j is computed; one
  // barrier per tile.  Unrolled by two so that every LDS offset is an
  // immediate.
  int pos = 0, kv = 0;
  auto advance = [&]() {  // next tile, moving to the next run when needed
    pos += C::BN;
    if (pos >= it.ke) {
      it.next_run();
      pos = it.ks;
    }
    kv = min(C::BN, it.ke - pos);
  };
  auto issue = [&](int buf) {
    blk.template issue<false>(buf, kbase, a.k_sn, pos, kv);
    blk.template issue<true>(buf, vbase, a.v_sn, pos, kv);
  };
  if (n_walk > 0) {
    it.next_run();
    pos = it.ks;
    kv = min(C::BN, it.ke - pos);
    issue(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // The loop is instantiated once per softmax mode; every wave of the
  // workgroup runs the same loads and barriers in either.
  auto run = [&](auto fixed_c) {
    constexpr bool F = decltype(fixed_c)::value;
    for (int i = 0; i + 1 < n_walk; i += 2) {
      const int kv0 = kv;
      advance();  // tile i+1 -> buffer 1
      issue(1);
      if (compute) blk.template tile<0, F>(kv0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int kv1 = kv;
      if (i + 2 < n_walk) {  // tile i+2 -> buffer 0
        advance();
        issue(0);
      }
      if (compute) blk.template tile<1, F>(kv1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if ((n_walk & 1) && compute) blk.template tile<0, F>(kv);
  };
  if (fixed)
    run(std::true_type{});
  else
    run(std::false_type{});

  // ---- a half writes its partial record (unnormalised O, partial row sum,
  // reference) for lvsa_combine, which runs after this kernel
  if (half >= 0) {
    if (compute) {
      constexpr int R4 = kPartialFloats(D) / 4;
      float4 *rec = reinterpret_cast<float4 *>(a.partial) +
                    ((int64_t)(slot * 2 + half) * NW + blk.wave) * R4 * 64 + blk.lane;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          rec[(i * 4 + j) * 64] = make_float4(blk.oacc[i][j * 4], blk.oacc[i][j * 4 + 1], blk.oacc[i][j * 4 + 2],
                                              blk.oacc[i][j * 4 + 3]);
      rec[(R4 - 1) * 64] = make_float4(blk.l_run, blk.m_run, 0.f, 0.f);
    }
    return;
  }

  // ---- epilogue: normalise, round to bf16, store
  {
    const int r = row0 + blk.l32;
    // both lane halves hold the same row: reduce before the early exit
    const float l_tot = swap_halves_sum(blk.l_run);
    if (r < P) {
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      u16 *op = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + ((int64_t)t * P + r) * a.o_sn;
#pragma unroll
      for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x4_t o4;
#pragma unroll
          for (int j = 0; j < 4; ++j) o4[j] = (__bf16)(blk.oacc[dc][i * 4 + j] * inv);
          *reinterpret_cast<bf16x4_t *>(op + dc * 32 + i * 8 + blk.hf * 4) = o4;
        }
    }
  }
}

// Largest key norm of one (b, h, frame): one workgroup per frame streams its
// P key rows once (16 bytes per lane, D/8 lanes per row) and writes
// max_j |k_j| (from fp32 sums of squares of the bf16 values) to
// knorm[(b·H + h)·T + t].  Workgroup 0 also zeroes the attention kernel's 8
// ticket counters.
template <int D>
__global__ __launch_bounds__(256) void lvsa_key_norms(const u16 *k, int64_t k_sb, int64_t k_sh, int32_t k_sn,
                                                      int32_t H, int32_t T, int32_t P, float *knorm, int *tickets) {
  if (blockIdx.x == 0 && threadIdx.x < kNumXcd)  // for the attention launch that follows
    __hip_atomic_store(tickets + threadIdx.x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  constexpr int LPR = D / 8;          // lanes per key row
  constexpr int RPI = 256 / LPR;      // rows per workgroup iteration
  const int item = blockIdx.x;        // (b·H + h)·T + t
  const int t = item % T;
  const int bh = item / T;
  const int h = bh % H;
  const int b = bh / H;
  const u16 *base = k + (int64_t)b * k_sb + (int64_t)h * k_sh + (int64_t)t * P * k_sn;
  const int col = (threadIdx.x % LPR) * 8;
  float best = 0.f;
  for (int r = threadIdx.x / LPR; r < P; r += RPI) {
    const bf16x8_t x = *reinterpret_cast<const bf16x8_t *>(base + (int64_t)r * k_sn + col);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf((float)x[e], (float)x[e], ss);
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);  // the row's LPR lanes
    best = fmaxf(best, ss);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = fmaxf(best, __shfl_xor(best, o));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) knorm[item] = __builtin_sqrtf(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
}

// Merges the two halves of every split item: one workgroup per record slot,
// one wave per 32 query rows as in lvsa_attn_fwd.  Each lane reads its two
// partial records (O accumulators, partial row sum l and reference m of its
// query), rescales both to the larger reference, adds, normalises and
// stores the item's output rows.  Runs after lvsa_attn_fwd on the same
// stream, so the records are complete.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void lvsa_combine(Args a) {
  const int x = blockIdx.x / a.split_cap, j = blockIdx.x % a.split_cap;
  int base, cnt;
  xcd_range(a.n_wg, x, &base, &cnt);
  const int S = split_count(a.split_cap, cnt);
  if (j >= S) return;
  const int item = base + (cnt - S) + j;
  const int qt = item % a.q_tiles;
  const int rest = item / a.q_tiles;
  const int t = rest % a.T;
  const int bh = rest / a.T;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = qt * NW * 32 + wave * 32;
  if (row0 >= a.P) return;  // a wave with no rows wrote no record
  constexpr int R4 = kPartialFloats(D) / 4;
  const float4 *r0 = reinterpret_cast<const float4 *>(a.partial) + ((int64_t)(blockIdx.x * 2) * NW + wave) * R4 * 64 + lane;
  const float4 *r1 = r0 + (int64_t)NW * R4 * 64;
  const float4 t0 = r0[(R4 - 1) * 64], t1 = r1[(R4 - 1) * 64];
  // weights 2^(m_h - m); a half that saw no key has m_h = -inf and weight 0
  const float m = fmaxf(t0.y, t1.y);
  const float w0 = t0.y == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(t0.y - m);
  const float w1 = t1.y == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(t1.y - m);
  const float l = w0 * t0.x + w1 * t1.x;
  const float l_tot = swap_halves_sum(l);
  const int r = row0 + (lane & 31);
  if (r >= a.P) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  u16 *op = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + ((int64_t)t * a.P + r) * a.o_sn;
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 o0 = r0[(dc * 4 + i) * 64], o1 = r1[(dc * 4 + i) * 64];
      bf16x4_t o4;
      o4[0] = (__bf16)((w0 * o0.x + w1 * o1.x) * inv);
      o4[1] = (__bf16)((w0 * o0.y + w1 * o1.y) * inv);
      o4[2] = (__bf16)((w0 * o0.z + w1 * o1.z) * inv);
      o4[3] = (__bf16)((w0 * o0.w + w1 * o1.w) * inv);
      *reinterpret_cast<bf16x4_t *>(op + dc * 32 + i * 8 + (lane >> 5) * 4) = o4;
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
  if (x->stride_n > (int64_t{1} << 24))
    return lvsa::fail(LVSA_ERR_SHAPE, "%s: stride_n above 2^24 elements is not supported", name);
  return LVSA_OK;
}

// Byte extent [lo, hi) touched by a tensor.
void extent(const lvsa_tensor *x, uintptr_t *lo, uintptr_t *hi) {
  const int64_t last = (x->B - 1) * x->stride_b + (x->H - 1) * x->stride_h + (x->N - 1) * x->stride_n + x->D;
  *lo = reinterpret_cast<uintptr_t>(x->data);
  *hi = *lo + (uintptr_t)last * 2;
}

// True if two distinct elements of x share an address.  Sorts the
// dimensions of size > 1 by stride and requires each stride to step past
// the whole extent of the smaller ones (the usual test for a strided layout
// without self-overlap; D is the contiguous innermost dimension).
bool self_overlapping(const lvsa_tensor *x) {
  int64_t st[3], sz[3];
  int n = 0;
  const int64_t dims[3][2] = {{x->stride_b, x->B}, {x->stride_h, x->H}, {x->stride_n, x->N}};
  for (const auto &d : dims)
    if (d[1] > 1) {
      st[n] = d[0];
      sz[n] = d[1];
      ++n;
    }
  for (int i = 1; i < n; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
      std::swap(st[j], st[j - 1]);
      std::swap(sz[j], sz[j - 1]);
    }
  int64_t extent = x->D;  // elements spanned by the dimensions placed so far
  for (int i = 0; i < n; ++i) {
    if (st[i] < extent) return true;
    extent = st[i] * (sz[i] - 1) + extent;
  }
  return false;
}

bool overlaps(const lvsa_tensor *a, const lvsa_tensor *b) {
  uintptr_t a0, a1, b0, b1;
  extent(a, &a0, &a1);
  extent(b, &b0, &b1);
  return a0 < b1 && b0 < a1;
}

template <int D, int NW>
int launch(const Args &args, hipStream_t stream) {
  if (args.knorm) {
    // the key-norm table first, on the same stream
    hipLaunchKernelGGL((lvsa_key_norms<D>), dim3(args.n_wg / args.q_tiles), dim3(256), 0, stream, args.k, args.k_sb,
                       args.k_sh, args.k_sn, args.H, args.T, args.P, const_cast<float *>(args.knorm), args.tickets);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return lvsa::fail(LVSA_ERR_HIP, "key-norm kernel launch failed: %s", hipGetErrorString(e));
  }
  // With tickets: one workgroup per ticket (items, plus one more per split
  // item), and 1/8 more, so that the fastest XCD can take over up to that
  // share of the others' items.
  const int64_t grid =
      args.tickets ? args.n_wg + (int64_t)kNumXcd * args.split_cap + args.n_wg / 8 + kNumXcd : args.n_wg;
  hipLaunchKernelGGL((lvsa_attn_fwd<D, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return lvsa::fail(LVSA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  if (args.tickets && args.split_cap > 0) {
    hipLaunchKernelGGL((lvsa_combine<D, NW>), dim3(kNumXcd * args.split_cap), dim3(NW * 64), 0, stream, args);
    e = hipGetLastError();
    if (e != hipSuccess) return lvsa::fail(LVSA_ERR_HIP, "combine kernel launch failed: %s", hipGetErrorString(e));
  }
  return lvsa::ok();
}

// Workspace: the key-norm table (B·H·T floats), then, at the next
// 256-byte boundary, the 8 ticket counters (256 bytes), then the partial
// records of the split items (8·split_cap slots × 2 halves × NW waves × 64
// lanes × kPartialFloats(D) floats).
constexpr int kSplitPerXcd = 96;  // items per XCD range run as two halves, at most
int64_t norms_bytes_for(int64_t B, int64_t H, int64_t T) {
  return ((B * H * T * (int64_t)sizeof(float) + 255) / 256) * 256;
}
int64_t items_for(int64_t B, int64_t H, int64_t N, int64_t T) {
  const int64_t P = N / T, BM = LVSA_NW * 32;
  return B * H * T * ((P + BM - 1) / BM);
}
// At most a quarter of every XCD range is split.
int32_t split_cap_for(int64_t items) { return (int32_t)std::min<int64_t>(kSplitPerXcd, items / (4 * kNumXcd)); }
int64_t workspace_bytes_for(int64_t B, int64_t H, int64_t N, int64_t D, int64_t T) {
  const int64_t partial =
      (int64_t)kNumXcd * split_cap_for(items_for(B, H, N, T)) * 2 * LVSA_NW * 64 * kPartialFloats((int)D) * 4;
  return norms_bytes_for(B, H, T) + 256 + partial;
}

int attention_impl(const lvsa_tensor *q, const lvsa_tensor *k, const lvsa_tensor *v,
                   const int32_t *row_ptr_dev, const int32_t *col_idx_dev, int32_t T, int32_t nnz,
                   lvsa_tensor *out, float scale, void *workspace, int64_t workspace_bytes, bool use_ws,
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
  if (self_overlapping(out))
    return lvsa::fail(LVSA_ERR_SHAPE, "out has overlapping elements (its strides alias two (b, h, token) rows)");
  if (T < 1) return lvsa::fail(LVSA_ERR_ARG, "T=%d: need T >= 1", T);
  if (q->N % T) return lvsa::fail(LVSA_ERR_SHAPE, "N=%lld is not a multiple of T=%d", (long long)q->N, T);
  if (q->N > INT32_MAX / 2) return lvsa::fail(LVSA_ERR_SHAPE, "N=%lld too large", (long long)q->N);
  if (!row_ptr_dev || !col_idx_dev || nnz < 0)
    return lvsa::fail(LVSA_ERR_ARG, "row_ptr/col_idx NULL or nnz < 0");
  {
    uint32_t bits;  // exponent all ones: inf or NaN (a bit test no fast-math flag can fold)
    std::memcpy(&bits, &scale, sizeof bits);
    if ((bits & 0x7f800000u) == 0x7f800000u) return lvsa::fail(LVSA_ERR_ARG, "scale is not finite");
  }
  if (use_ws) {
    const int64_t need = workspace_bytes_for(q->B, q->H, q->N, q->D, T);
    if (!workspace) return lvsa::fail(LVSA_ERR_ARG, "workspace is NULL");
    // the partial records are written and read 16 bytes at a time
    if (reinterpret_cast<uintptr_t>(workspace) % 16) return lvsa::fail(LVSA_ERR_ARG, "workspace not 16-byte aligned");
    if (workspace_bytes < need)
      return lvsa::fail(LVSA_ERR_CAPACITY, "workspace of %lld bytes < required %lld", (long long)workspace_bytes,
                        (long long)need);
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace), w1 = w0 + (uintptr_t)need;
    for (const lvsa_tensor *x : {q, k, v, (const lvsa_tensor *)out}) {
      uintptr_t x0, x1;
      extent(x, &x0, &x1);
      if (w0 < x1 && x0 < w1) return lvsa::fail(LVSA_ERR_ARG, "workspace overlaps a tensor");
    }
  }
  int dev;
  if ((rc = check_device(&dev))) return rc;

  const int D = (int)q->D;
  const int P = (int)(q->N / T);
  constexpr int NW = LVSA_NW;
  const int BM = NW * 32;
  const int q_tiles = (P + BM - 1) / BM;
  const int64_t n_wg = (int64_t)q->B * q->H * T * q_tiles;
  if (n_wg > INT32_MAX / 2) return lvsa::fail(LVSA_ERR_SHAPE, "grid of %lld workgroups too large", (long long)n_wg);

  Args a;
  a.q = static_cast<const u16 *>(q->data);
  a.k = static_cast<const u16 *>(k->data);
  a.v = static_cast<const u16 *>(v->data);
  a.o = static_cast<u16 *>(out->data);
  a.q_sb = q->stride_b; a.q_sh = q->stride_h; a.q_sn = (int32_t)q->stride_n;
  a.k_sb = k->stride_b; a.k_sh = k->stride_h; a.k_sn = (int32_t)k->stride_n;
  a.v_sb = v->stride_b; a.v_sh = v->stride_h; a.v_sn = (int32_t)v->stride_n;
  a.o_sb = out->stride_b; a.o_sh = out->stride_h; a.o_sn = (int32_t)out->stride_n;
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
  a.knorm = use_ws ? static_cast<const float *>(workspace) : nullptr;
  a.tickets = use_ws ? reinterpret_cast<int *>(static_cast<char *>(workspace) + norms_bytes_for(q->B, q->H, T))
                     : nullptr;
  a.partial = use_ws ? reinterpret_cast<float *>(static_cast<char *>(workspace) + norms_bytes_for(q->B, q->H, T) + 256)
                     : nullptr;
  a.split_cap = use_ws ? split_cap_for(n_wg) : 0;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) return launch<128, NW>(a, s);
  return launch<64, NW>(a, s);
}

}  // namespace

extern "C" int lvsa_attention(const lvsa_tensor *q, const lvsa_tensor *k, const lvsa_tensor *v,
                              const int32_t *row_ptr_dev, const int32_t *col_idx_dev,
                              int32_t T, int32_t nnz, lvsa_tensor *out, float scale,
                              void *stream) {
  return attention_impl(q, k, v, row_ptr_dev, col_idx_dev, T, nnz, out, scale, nullptr, 0, false, stream);
}

extern "C" int lvsa_attention_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t T,
                                              int64_t *bytes) {
  if (!bytes) return lvsa::fail(LVSA_ERR_ARG, "bytes is NULL");
  if (B < 1 || H < 1 || T < 1 || N < 1) return lvsa::fail(LVSA_ERR_ARG, "B, H, N and T must be >= 1");
  if (D != 64 && D != 128) return lvsa::fail(LVSA_ERR_SHAPE, "D=%lld, supported 64 and 128", (long long)D);
  if (N % T) return lvsa::fail(LVSA_ERR_SHAPE, "N=%lld is not a multiple of T=%d", (long long)N, T);
  if (N > INT32_MAX / 2 || B * H > (int64_t{1} << 40) / N)
    return lvsa::fail(LVSA_ERR_ARG, "B*H*N too large");
  *bytes = workspace_bytes_for(B, H, N, D, T);
  return lvsa::ok();
}

extern "C" int lvsa_attention_ws(const lvsa_tensor *q, const lvsa_tensor *k, const lvsa_tensor *v,
                                 const int32_t *row_ptr_dev, const int32_t *col_idx_dev,
                                 int32_t T, int32_t nnz, lvsa_tensor *out, float scale,
                                 void *workspace, int64_t workspace_bytes, void *stream) {
  return attention_impl(q, k, v, row_ptr_dev, col_idx_dev, T, nnz, out, scale, workspace, workspace_bytes, true,
                        stream);
}
