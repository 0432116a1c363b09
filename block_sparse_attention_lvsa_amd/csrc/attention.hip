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
// Two kernels, one per kind of work item (bf16 MFMA, fp32 accumulation):
//
//   lvsa_attn_span (frames of at least 384 tokens: every video workload).
//   A work item is the 384 consecutive query tokens [384·i, 384·i + 384) of
//   one (b, h); a workgroup is 8 waves of 48 rows, one per CU (2 waves per
//   SIMD), so every K/V tile brought into LDS serves 384 rows.  Each wave
//   computes its rows as three 16-row blocks with v_mfma_f32_16x16x32_bf16:
//   every K and Vᵀ operand read from LDS feeds the MFMAs of all three blocks.
//   An item may cross one frame boundary: it then walks the union of the two
//   frames' key lists, and each wave computes only the key frames its rows
//   attend -- a wave whose rows straddle the boundary masks, per row, the
//   frames only one of its two frames attends.
//
//   lvsa_attn_frame (shorter frames).  A work item is 128 rows of one frame;
//   a workgroup is 4 waves of 32 rows (3 workgroups per CU), with
//   v_mfma_f32_32x32x16_bf16.
//
// Key iteration.  The walk merges consecutive key frames with the same
// membership into segments: tokens are frame-major, so frames [f0, f1] are
// the one contiguous token range [f0·P, (f1+1)·P).  Each segment is
// streamed in tiles of 32 keys; only the last tile of a segment is partial,
// and its missing keys are masked.
//
// Per key tile, per wave (all on the matrix cores):
//   Sᵀ = K · Qᵀ     K from LDS, Q held in VGPRs for the whole walk.
//   Softmax in the log2 domain, per query row: with a lazily updated running
//   max (rescale only when the tile max exceeds it by more than 2^8, so exp2
//   arguments stay <= 8 and fp32 cannot overflow); or, given per-frame key
//   norms, a fixed reference from a Cauchy-Schwarz bound, subtracted by
//   starting the Q·Kᵀ chains from it.
//   Oᵀ += Vᵀ · P    P (bf16) comes straight from the Sᵀ accumulator
//                   registers; the Vᵀ operand is built by transposing LDS
//                   reads (ds_read_b64_tr_b16).
//
// K/V staging.  Each tile's K and V rows go from global memory straight into
// LDS (buffer loads with the LDS-destination bit, 16 bytes per lane), double
// buffered: the loads of tile j+1 run while tile j is computed, one
// workgroup barrier per tile.  16-byte chunks are XOR-swizzled by key so
// every MFMA operand read is bank-conflict free.
//
// Launch order.  Workgroups are dispatched round-robin over the 8 XCDs; each
// XCD receives a contiguous range of work items (in token order): the query
// tiles of a frame and neighbouring frames (which share most of their key
// frames) run on the same XCD and hit in its L2.  With a workspace the
// items are taken from per-XCD counters, so XCDs that clock faster take over
// work from slower ones (take_item).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <utility>

#include "lvsa_internal.h"

// Device scratch of lvsa_attention_ws_static, for callers that cannot
// allocate: the key-norm table, the work counters and the partial records of
// lvsa_attention_ws, at most kStaticScratchBytes.  Every GPU the library runs
// on holds its own copy until the process ends.  Host code never uses this
// name as a device address: it takes the address per device from
// hipGetSymbolAddress (static_scratch_ptr below).
static constexpr int64_t kStaticScratchBytes = LVSA_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

// Tuning knobs of the frame kernel (compile-time): the register budget
// expressed as resident waves per SIMD, keys per tile, and how many K
// operand reads run ahead of the Q·Kᵀ MFMA chain.
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
constexpr int kFrameWaves = 4;      // waves per workgroup of the frame kernel
constexpr int kSpanRows = 384;      // query rows per work item of the span kernel
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
  // range run as two halves of their key walk, whose partial results
  // (records of kPartialFloats(D) or kSpanPartialFloats(D) floats per lane,
  // slot x·split_cap + j) go to `partial` and are merged by the combine
  // kernel; split_cap = 0 splits nothing.
  float *partial;
  int32_t split_cap;
};

// Read-only kernel inputs read at wave-uniform addresses go through the
// constant address space, so they become scalar loads served by the scalar
// cache instead of vector loads that each wait for memory.
typedef const __attribute__((address_space(4))) int32_t *const_i32p;
typedef const __attribute__((address_space(4))) float *const_f32p;

// The key walk of a workgroup whose query rows lie in frames t0 and t1
// (t1 = t0, or t0 + 1 when the rows cross a frame boundary): the union of
// the two CSR rows, in ascending frame order, as segments of consecutive
// frames with the same membership (bit 0: the frame is in A(t0), bit 1: in
// A(t1); with one row both bits are set).  Tokens are frame-major, so a
// segment of frames [f0, f1] is the one contiguous token range
// [f0·P, (f1+1)·P).  Frames at or above f_hi are not walked.
//
// Each row's entries are read in order; an entry outside [0, T), or not
// above the last entry taken from its row, is skipped, so a malformed row
// never causes an out-of-range read and never repeats a frame.  Every value
// is wave-uniform (scalar registers; the state is kept small, since the
// main loop's scalar registers are scarce).
struct SegIter {
  const_i32p cols;
  int32_t T, P, f_hi;
  int32_t e0, end0, last0;  // row of t0: next entry, end, last frame taken
  int32_t e1, end1, last1;  // row of t1 (no entries when the walk has one row)
  int32_t bits0;            // membership of a frame of row t0: 1, or 3 with one row
  int32_t ks, ke, mem;

  // The next frame row 0 (row 1) keeps, or T when it has none left.
  __device__ int32_t peek0() {
    while (e0 < end0) {
      const int32_t f = cols[e0];
      if (f > last0 && f < T) return f;
      ++e0;
    }
    return T;
  }
  __device__ int32_t peek1() {
    while (e1 < end1) {
      const int32_t f = cols[e1];
      if (f > last1 && f < T) return f;
      ++e1;
    }
    return T;
  }
  // Takes frame f from the rows whose next frame it is; returns its membership.
  __device__ int take(int32_t f, int32_t a0, int32_t a1) {
    int m = 0;
    if (a0 == f) {
      last0 = f;
      ++e0;
      m = bits0;
    }
    if (a1 == f) {
      last1 = f;
      ++e1;
      m |= 2;
    }
    return m;
  }
  // Skips every frame below f_lo (the second half of a split walk).
  __device__ void skip_below(int32_t f_lo) {
    for (int32_t f; (f = peek0()) < f_lo;) take(f, f, T);
    for (int32_t f; (f = peek1()) < f_lo;) take(f, T, f);
  }
  __device__ bool next() {
    int32_t a0 = peek0(), a1 = peek1();
    const int32_t fs = min(a0, a1);
    if (fs >= f_hi) return false;
    const int m = take(fs, a0, a1);
    int32_t fe = fs;
    while (fe + 1 < f_hi) {
      a0 = peek0();
      a1 = peek1();
      const int mm = (a0 == fe + 1 ? bits0 : 0) | (a1 == fe + 1 ? 2 : 0);
      if (mm != m) break;
      take(fe + 1, a0, a1);
      ++fe;
    }
    ks = fs * P;
    ke = (fe + 1) * P;
    mem = m;
    return true;
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
  static constexpr int LOADS_PER_WAVE = LOADS >= NW ? LOADS / NW : 1;
  static constexpr int NLOADERS = LOADS / LOADS_PER_WAVE;  // waves that issue the tile loads
  // The loading waves are the last NLOADERS of the workgroup.  The sequencer
  // favours older waves, so after each barrier the oldest wave of every SIMD
  // goes straight to its matrix work while the younger ones issue the next
  // tile's loads (measured 1-2% faster than loads from the first waves;
  // fewer loading waves with more loads each was 5-7% slower).
  static constexpr int FIRST_LOADER = NW - NLOADERS;
  static constexpr int VSW = CH / 4;          // V swizzle step
  static constexpr int KEYS_PER_LOAD = 64 / CH;       // keys per 1 KB wave load
  static constexpr int STAGES = 2;                    // LDS tile buffers (loads run one tile ahead)
  static constexpr int LDS_BYTES = STAGES * 2 * TILE_BYTES; // {K, V} × STAGES
  static_assert(LOADS % NW == 0 || NW > LOADS, "tile loads must split evenly over the loading waves");
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

  // LDS tile buffers 0 and 1, {K, V} each.  Two arrays rather than one, so
  // the compiler sees that the direct-to-LDS loads into one buffer cannot
  // touch the other and does not wait for them before the tile's V reads.
  char *lds0, *lds1;
  __device__ __forceinline__ char *bufp(int buf) const { return buf ? lds1 : lds0; }
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

  static constexpr int kTileOffK = 0;             // within a buffer
  static constexpr int kTileOffV = C::TILE_BYTES;

  __device__ __forceinline__ void init_offsets(int32_t k_sn, int32_t v_sn) {
    // Load i of loading wave lw covers keys key0 + i·KEYS_PER_LOAD (one per
    // group of CH lanes); each lane writes stored chunk `pchunk` of its key's
    // row, which holds logical chunk pchunk ^ swizzle(key).
    const int lw = max(wave - C::FIRST_LOADER, 0);
    const int key0 = lw * C::LOADS_PER_WAVE * C::KEYS_PER_LOAD + lane / C::CH;
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
    const int lw = wave - C::FIRST_LOADER;
    if (lw < 0) return;  // wave-uniform
    char *dst = bufp(buf) + (IS_V ? kTileOffV : kTileOffK) + lw * C::LOADS_PER_WAVE * 1024;
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
    const char *Kb = bufp(KBUF) + kTileOffK;
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
    const char *Vb = bufp(VBUF) + kTileOffV;
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

// A work item's query rows.  SPAN = false: query tile qt (BM rows) of frame
// t of (b, h), items ordered (b, h, t, qt).  SPAN = true (frames of at least
// BM tokens): rows [qt·BM, qt·BM + BM) of the (b, h) token sequence, items
// ordered (b, h, qt); such a tile lies in frame t0 and possibly t1 = t0 + 1.
struct Item {
  int b, h, bh, t0, t1, tok0, tok_end;
};

template <int BM, bool SPAN>
__device__ __forceinline__ Item decode_item(const Args &a, int item) {
  Item it;
  const int qt = item % a.q_tiles;
  const int rest = item / a.q_tiles;
  if (SPAN) {
    it.bh = rest;
    it.tok0 = qt * BM;
    it.tok_end = min(a.T * a.P, it.tok0 + BM);
    it.t0 = it.tok0 / a.P;
    it.t1 = (it.tok_end - 1) / a.P;
  } else {
    const int t = rest % a.T;
    it.bh = rest / a.T;
    it.tok0 = t * a.P + qt * BM;
    it.tok_end = (t + 1) * a.P;
    it.t0 = it.t1 = t;
  }
  it.h = it.bh % a.H;
  it.b = it.bh / a.H;
  return it;
}

// ---- work items.  The items are split into 8 contiguous ranges, one per
// XCD, so that the query tiles of a frame and neighbouring frames (which
// share most key frames) run on one XCD and share its L2.  Statically,
// workgroup i runs the (i div 8)-th item of XCD i mod 8's range (the
// dispatcher deals workgroups round-robin over the XCDs).  With ticket
// counters, a workgroup takes the next item of the range of the XCD it runs
// on, and once that range is used up, of the others: the XCDs of one part
// run at different speeds (up to ~7% apart), and a static split leaves the
// fast ones idle while the slowest finishes.  More workgroups than items are
// launched; the ones that find no item left exit (returns false: uniform,
// all waves leave).
//
// The item (and, for a half, which half and its record slot) is broadcast
// through s_item, the first words of LDS tile buffer 1: the first tile loads
// (buffer 0) do not touch them, and every wave reads them before the barrier
// that precedes the loads into buffer 1.  (A separate __shared__ word
// measured 2.5-6% slower, from the code it changes.)
__device__ __forceinline__ bool take_item(const Args &a, int *s_item, int *item, int *half, int *slot) {
  if (a.tickets) {
    if (threadIdx.x == 0) {
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
    *item = __builtin_amdgcn_readfirstlane(s_item[0]);
    *half = __builtin_amdgcn_readfirstlane(s_item[1]);
    *slot = __builtin_amdgcn_readfirstlane(s_item[2]);
    return *item >= 0;
  }
  const int x = blockIdx.x % kNumXcd, j = blockIdx.x / kNumXcd;
  int base, cnt;
  xcd_range(a.n_wg, x, &base, &cnt);
  *item = base + j;
  *half = -1;
  *slot = 0;
  return true;
}

// The entries [rb, re) of CSR row t, offsets clamped to [0, nnz].
__device__ __forceinline__ void row_range(const Args &a, int t, int32_t *rb, int32_t *re) {
  const const_i32p rp = (const_i32p)a.row_ptr;
  int32_t b = rp[t], e = rp[t + 1];
  b = b < 0 ? 0 : (b > a.nnz ? a.nnz : b);
  e = e < b ? b : (e > a.nnz ? a.nnz : e);
  *rb = b;
  *re = e;
}

// The key walk of work item wi: the union of the CSR rows of its frames t0
// and t1 (one row when t1 = t0), split at frame fm for the two halves of a
// split item: the first half walks the frames below fm, the second the rest,
// so that together they walk exactly what the whole walk does.  fm is the
// middle entry of t0's row (any frame partitions the walk; the middle one
// halves it for well-formed rows).
__device__ __forceinline__ SegIter make_walk(const Args &a, const Item &wi, int half) {
  const bool two = wi.t1 != wi.t0;
  SegIter it;
  it.cols = (const_i32p)a.col_idx;
  it.T = a.T;
  it.P = a.P;
  it.f_hi = a.T;
  row_range(a, wi.t0, &it.e0, &it.end0);
  if (two)
    row_range(a, wi.t1, &it.e1, &it.end1);
  else
    it.e1 = it.end1 = 0;
  it.last0 = it.last1 = -1;
  it.bits0 = two ? 1 : 3;
  it.ks = it.ke = it.mem = 0;
  if (half >= 0) {
    const int32_t mid = it.e0 + (it.end0 - it.e0) / 2;
    int32_t fm = it.end0 > it.e0 ? it.cols[mid] : 0;
    fm = fm < 0 ? 0 : (fm > a.T ? a.T : fm);
    if (half == 0)
      it.f_hi = fm;
    else
      it.skip_below(fm);
  }
  return it;
}

// Tiles of bn keys in a walk.
__device__ __forceinline__ int walk_tiles(SegIter c, int bn) {
  int n = 0;
  while (c.next()) n += (c.ke - c.ks + bn - 1) / bn;
  return n;
}

// The largest key norm over the frames of wi's rows, from the per-frame
// table knorm: every entry of both rows, so that both halves of a split item
// decide alike.
__device__ __forceinline__ float walk_key_norm(const Args &a, const Item &wi) {
  const const_f32p fn = (const_f32p)(a.knorm + (int64_t)wi.bh * a.T);
  const const_i32p cols = (const_i32p)a.col_idx;
  float kn = 0.f;
  for (int r = 0; r < (wi.t1 != wi.t0 ? 2 : 1); ++r) {
    int32_t rb, re;
    row_range(a, r ? wi.t1 : wi.t0, &rb, &re);
    for (int32_t e = rb; e < re; ++e) {
      const int32_t f = cols[e];
      if (f >= 0 && f < a.T) kn = fmaxf(kn, fn[f]);
    }
  }
  return kn;
}

template <int D>
__global__ __launch_bounds__(kFrameWaves * 64)
__attribute__((amdgpu_waves_per_eu(LVSA_WAVES_PER_SIMD, LVSA_WAVES_PER_SIMD))) void lvsa_attn_frame(Args a) {
  constexpr int NW = kFrameWaves;
  using C = Cfg<D, NW>;
  __shared__ __attribute__((aligned(1024))) char lds0[C::LDS_BYTES / 2];  // K0 V0
  __shared__ __attribute__((aligned(1024))) char lds1[C::LDS_BYTES / 2];  // K1 V1

  Block<D, NW> blk;
  blk.lds0 = lds0;
  blk.lds1 = lds1;
  const int tid = threadIdx.x;
  blk.lane = tid & 63;
  blk.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  blk.l32 = blk.lane & 31;
  blk.hf = blk.lane >> 5;
  blk.scale_log2 = a.scale_log2;

  int item, half, slot;
  if (!take_item(a, reinterpret_cast<int *>(lds1), &item, &half, &slot)) return;
  const Item wi = decode_item<C::BM, false>(a, item);
  const u16 *kbase = a.k + (int64_t)wi.b * a.k_sb + (int64_t)wi.h * a.k_sh;
  const u16 *vbase = a.v + (int64_t)wi.b * a.v_sb + (int64_t)wi.h * a.v_sh;

  // ---- Q fragments: the wave's 32 rows × D, B-operand layout
  const int row0 = wi.tok0 + blk.wave * 32;  // token of the wave's first row
  const int my_row = row0 + blk.l32;
  {
    const bool ok = my_row < wi.tok_end;
    const u16 *qp = a.q + (int64_t)wi.b * a.q_sb + (int64_t)wi.h * a.q_sh + (int64_t)(ok ? my_row : 0) * a.q_sn +
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
  blk.m_run = -FLT_MAX;
  blk.l_run = 0.f;
  blk.init_offsets(a.k_sn, a.v_sn);
  // Whether the wave has rows in the tile (the last tile of a frame or of
  // the sequence may not fill every wave), as a scalar, so the per-tile test
  // is a scalar branch rather than a vector compare.
  const int compute = __builtin_amdgcn_readfirstlane(row0 < wi.tok_end ? 1 : 0);

  // ---- the key walk: the CSR row of the item's frame
  SegIter it = make_walk(a, wi, half);
  const int n_walk = walk_tiles(it, C::BN);  // tiles this workgroup walks

  // ---- softmax reference.  Without a key-norm table: the running max,
  // raised lazily.  With one: by Cauchy-Schwarz every score of query i lies
  // within ±|q_i|·K, K the largest key norm over the walk's frames, so
  // R_i = scale·log2e·|q_i|·K·(1 + 2^-8) bounds every exponent (the factor
  // covers the rounding of the fp32 norms and of the MFMA dot products).  A
  // wave whose lanes all have 2·R_i <= kMaxRefGap (the bound cannot sit more
  // than 2·R_i above a row's true maximum) takes R_i as a fixed reference:
  // no running max, no rescale, and the subtraction is folded into the
  // Q·Kᵀ chain's initial accumulator.  Other waves keep the running max.
  bool fixed = false;
  if (a.knorm) {
    const float kn = walk_key_norm(a, wi);
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
  auto advance = [&]() {  // next tile, moving to the next segment when needed
    pos += C::BN;
    if (pos >= it.ke) {
      it.next();
      pos = it.ks;
    }
    kv = min(C::BN, it.ke - pos);
  };
  auto issue = [&](int buf) {
    blk.template issue<false>(buf, kbase, a.k_sn, pos, kv);
    blk.template issue<true>(buf, vbase, a.v_sn, pos, kv);
  };
  if (n_walk > 0) {
    it.next();
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
    auto step = [&](auto buf_c, int kvj) {
      if (compute) blk.template tile<decltype(buf_c)::value, F>(kvj);
    };
    for (int i = 0; i + 1 < n_walk; i += 2) {
      const int kv0 = kv;
      advance();  // tile i+1 -> buffer 1
      issue(1);
      step(std::integral_constant<int, 0>{}, kv0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int kv1 = kv;
      if (i + 2 < n_walk) {  // tile i+2 -> buffer 0
        advance();
        issue(0);
      }
      step(std::integral_constant<int, 1>{}, kv1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if (n_walk & 1) step(std::integral_constant<int, 0>{}, kv);
  };
  if (fixed)
    run(std::true_type{});
  else
    run(std::false_type{});

  // ---- a half writes its partial record (unnormalised O, partial row sum,
  // reference) for lvsa_combine_frame, which runs after this kernel
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
    // both lane halves hold the same row: reduce before the early exit
    const float l_tot = swap_halves_sum(blk.l_run);
    if (my_row < wi.tok_end) {
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      u16 *op = a.o + (int64_t)wi.b * a.o_sb + (int64_t)wi.h * a.o_sh + (int64_t)my_row * a.o_sn;
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
// one wave per 32 query rows as in lvsa_attn_frame.  Each lane reads its two
// partial records (O accumulators, partial row sum l and reference m of its
// query), rescales both to the larger reference, adds, normalises and
// stores the item's output rows.  Runs after lvsa_attn_frame on the same
// stream, so the records are complete.
template <int D>
__global__ __launch_bounds__(kFrameWaves * 64) void lvsa_combine_frame(Args a) {
  constexpr int NW = kFrameWaves;
  const int x = blockIdx.x / a.split_cap, j = blockIdx.x % a.split_cap;
  int base, cnt;
  xcd_range(a.n_wg, x, &base, &cnt);
  const int S = split_count(a.split_cap, cnt);
  if (j >= S) return;
  const Item wi = decode_item<NW * 32, false>(a, base + (cnt - S) + j);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = wi.tok0 + wave * 32;
  if (row0 >= wi.tok_end) return;  // a wave with no rows wrote no record
  constexpr int R4 = kPartialFloats(D) / 4;
  const float4 *r0 = reinterpret_cast<const float4 *>(a.partial) + ((int64_t)(blockIdx.x * 2) * NW + wave) * R4 * 64 + lane;
  const float4 *r1 = r0 + (int64_t)NW * R4 * 64;
  const float4 t0 = r0[(R4 - 1) * 64], t1 = r1[(R4 - 1) * 64];
  // weights 2^(m_h - m); a half that saw no key of a row has l_h = 0 and
  // m_h = -FLT_MAX (its start), so its weight is 0 unless neither half saw
  // one (then l = 0 and the row is zero)
  const float m = fmaxf(t0.y, t1.y);
  const float w0 = __builtin_amdgcn_exp2f(t0.y - m);
  const float w1 = __builtin_amdgcn_exp2f(t1.y - m);
  const float l = w0 * t0.x + w1 * t1.x;
  const float l_tot = swap_halves_sum(l);
  const int r = row0 + (lane & 31);
  if (r >= wi.tok_end) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  u16 *op = a.o + (int64_t)wi.b * a.o_sb + (int64_t)wi.h * a.o_sh + (int64_t)r * a.o_sn;
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

// ------------------------------------------------------------ span kernel --
// Frames of at least kSpanRows tokens (every video workload).  A workgroup
// is 8 waves, one per CU (2 waves per SIMD), over the kSpanRows consecutive
// query tokens of a work item; each wave owns 48 rows as three 16-row
// blocks and uses v_mfma_f32_16x16x32_bf16, so that every K operand read
// from LDS feeds the Q·Kᵀ MFMAs of all three blocks and every Vᵀ operand
// read the P·V MFMAs of all three: a third fewer LDS bytes per flop than
// waves of 32 rows with the 32x32x16 MFMA.
//
// Lane layouts of v_mfma_f32_16x16x32_bf16 (64 lanes, l = 16g + s):
//   A (16 x 32): lane l holds A[s][8g + e], e = 0..7 (8 bf16)
//   B (32 x 16): lane l holds B[8g + e][s]
//   C (16 x 16): lane l holds C[4g + r][s], r = 0..3 (4 fp32)
// Per tile of 32 keys, per wave:
//   Sᵀ(16 keys × 16 queries), for 2 key blocks × 3 query blocks: A = K rows
//     (key 16kbk + s, dims 32dc + 8g + e), B = the wave's Q rows (held in
//     VGPRs), D/32 reduction steps; lane l then holds query 16qb + s and
//     keys 16kbk + 4g + r, so a query's row lies in lanes s, s+16, s+32,
//     s+48 (row reductions: two lane swaps).
//   P (bf16) of query block qb is the B operand of P·V as it stands: k-slot
//     8g + 4kbk + r is key 16kbk + 4g + r.
//   Oᵀ(16 dims × 16 queries) += Vᵀ · P for D/16 dim blocks × 3 query blocks;
//     the Vᵀ operand (dim 16db + s, the same eight keys per lane as P's
//     k-slots) comes from two transposing LDS reads of four keys each.
//   The row sums, one more MFMA per query block with a block of ones as the
//     A operand: every element of its accumulator is the row's sum of P.
//     Vector and matrix instructions of a SIMD largely take turns, and this
//     trades 12 vector instructions per wave and tile for 3 MFMAs (1.6-2.1%
//     faster than summing with v_dot2c).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kQB = 3;  // 16-row query blocks per wave
// Floats per lane in a partial record of the span kernel: the lane's Oᵀ
// accumulators (3 × D/16 × 4), the three row sums (in the lanes of g = 0,
// zero in the others, so that a sum over a row's four lanes gives them) and
// references, padding to 16 bytes.
__host__ __device__ constexpr int kSpanPartialFloats(int d) { return kQB * d / 4 + 8; }

template <int D>
struct SpanCfg {
  static constexpr int NW = 8;                  // waves per workgroup (2 per SIMD)
  static constexpr int BM = NW * 16 * kQB;      // query rows per workgroup
  static_assert(BM == kSpanRows, "work item size");
  static constexpr int BN = 32;                 // keys per LDS tile
  static constexpr int CH = D / 8;              // 16-byte chunks per key row
  static constexpr int ROWB = D * 2;            // bytes per key row
  static constexpr int TILE_BYTES = BN * ROWB;
  static constexpr int LOADS = TILE_BYTES / 1024;  // 1 KB wave loads per tile
  // The loads are issued by the last four waves, the younger wave of each
  // SIMD, so that the older one goes straight to its matrix work after a
  // barrier (the sequencer favours older waves): measured 1-2% faster than
  // one load of each per wave from all eight.
  static constexpr int LOADS_PER_WAVE = LOADS >= 4 ? LOADS / 4 : 1;
  static constexpr int NLOADERS = LOADS / LOADS_PER_WAVE;
  static constexpr int FIRST_LOADER = NW - NLOADERS;
  static constexpr int VSW = CH / 4;            // V swizzle step
  static constexpr int KEYS_PER_LOAD = 64 / CH;
  static constexpr int DC = D / 32;             // 32-dim reduction steps of Q·Kᵀ
  static constexpr int DB = D / 16;             // 16-dim blocks of O
  static constexpr int LDS_BYTES = 2 * 2 * TILE_BYTES;  // {K, V} × 2 buffers
  static_assert(LOADS % LOADS_PER_WAVE == 0 && NLOADERS <= NW, "tile loads must split evenly over the loading waves");
};

__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
// Max and sum over the four lanes s, s+16, s+32, s+48 that hold one query
// row of a 16x16 accumulator.
__device__ __forceinline__ float row4_max(float x) { return swap_halves_max(xor16_max(x)); }
__device__ __forceinline__ float row4_sum(float x) { return swap_halves_sum(xor16_sum(x)); }

// One wave's state and steps in the span kernel (48 query rows).  LDS tile
// layout: K chunk c of key j at c ^ (j mod CH), as in the frame kernel; V
// chunk c at c ^ vswz(j).  The transposing Vᵀ reads of a 32-lane half read
// keys 4g + 0..3 for g = 0, 1 (or 2, 3) at the same dims; the term in bit
// 2 of the key puts those key groups into different banks (without it,
// 2-way conflicts on every Vᵀ read: 0.5-0.6% slower).
template <int D>
struct SpanBlock {
  using C = SpanCfg<D>;
  static __device__ __forceinline__ int vswz(int j) { return C::VSW * (j & 3) ^ (C::VSW / 2) * ((j >> 2) & 1); }
  char *lds0, *lds1;  // tile buffers 0 and 1, {K, V} each (separate arrays, as in Block)
  __device__ __forceinline__ char *bufp(int buf) const { return buf ? lds1 : lds0; }
  int lane, wave, s16, g;  // lane = 16g + s16
  float scale_log2;
  bf16x8_t qf[kQB][C::DC];   // Q rows, B operand: query 16qb + s16, dims 32dc + 8g + e
  f32x4_t oacc[kQB][C::DB];  // Oᵀ blocks: dims 16db + 4g + r of query 16qb + s16
  f32x4_t bias[kQB];         // with a fixed reference R: -R, the Q·Kᵀ chains' initial value
  float m_run[kQB];    // per query block: the softmax reference (log2 domain)
  f32x4_t lsum[kQB];  // per query block: the row sums of P (all four elements alike)
  int32_t kro[C::DC], vro[C::DB];  // LDS byte offsets of this lane's K and Vᵀ operands
  int32_t koffb[C::LOADS_PER_WAVE], voffb[C::LOADS_PER_WAVE];  // load byte offsets
  static constexpr int kTileOffK = 0;  // within a buffer
  static constexpr int kTileOffV = C::TILE_BYTES;

  __device__ __forceinline__ void init_offsets(int32_t k_sn, int32_t v_sn) {
    const int lw = max(wave - C::FIRST_LOADER, 0);
    const int key0 = lw * C::LOADS_PER_WAVE * C::KEYS_PER_LOAD + lane / C::CH;
    const int pchunk = lane % C::CH;
#pragma unroll
    for (int i = 0; i < C::LOADS_PER_WAVE; ++i) {
      const int key = key0 + i * C::KEYS_PER_LOAD;
      koffb[i] = (key * k_sn + (pchunk ^ (key & (C::CH - 1))) * 8) * 2;
      voffb[i] = (key * v_sn + (pchunk ^ vswz(key)) * 8) * 2;
    }
    // K operand of key block kbk: key 16kbk + s16 (kbk adds an immediate 16
    // rows: the swizzle depends on the key modulo CH only), logical chunk 4dc + g
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) kro[dc] = s16 * C::ROWB + (((4 * dc + g) ^ (s16 & (C::CH - 1))) * 16);
    // Vᵀ operand of dim block db, transposing reads: source lane s16 points at
    // key 4g + s16/4 (+16 for the second read) and dims 16db + 4(s16 mod 4)..+3
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int c = 2 * db + ((s16 & 3) >> 1);
      vro[db] = (4 * g + (s16 >> 2)) * C::ROWB + ((c ^ vswz(4 * g + (s16 >> 2))) * 16) + (s16 & 1) * 8;
    }
  }

  template <bool IS_V>
  __device__ __forceinline__ void issue(int buf, const u16 *base, int32_t sn, int pos, int kv) {
    const u16 *tb = base + (int64_t)pos * sn;
    const int nrec = ((kv - 1) * sn + D) * 2;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)tb, 0, nrec, kBufferFlags);
    const int lw = wave - C::FIRST_LOADER;
    if (lw < 0) return;
    char *dst = bufp(buf) + (IS_V ? kTileOffV : kTileOffK) + lw * C::LOADS_PER_WAVE * 1024;
#pragma unroll
    for (int i = 0; i < C::LOADS_PER_WAVE; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + i * 1024), 16, IS_V ? voffb[i] : koffb[i], 0, 0, 0);
  }

  // The first K operand reads of a tile (reduction step 0, both key blocks),
  // issued right after the barrier, ahead of the walk's scalar work.
  template <int KBUF>
  __device__ __forceinline__ void kpre(bf16x8_t (&kp)[2]) const {
    const char *Kb = bufp(KBUF) + kTileOffK;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) kp[kbk] = *(const lds_bf16x8 *)(Kb + kro[0] + kbk * 16 * C::ROWB);
  }
  // Sᵀ blocks (2 key blocks × 3 query blocks) of the K tile in buffer KBUF;
  // with a fixed reference (FIXED) the chains start from -R (Q pre-scaled).
  template <int KBUF, bool FIXED>
  __device__ __forceinline__ void qk(f32x4_t (&sc)[2][kQB], const bf16x8_t (&kp)[2]) const {
    const char *Kb = bufp(KBUF) + kTileOffK;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) sc[kbk][qb] = FIXED ? bias[qb] : f32x4_t{};
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
        const bf16x8_t kf = dc == 0 ? kp[kbk] : *(const lds_bf16x8 *)(Kb + kro[dc] + kbk * 16 * C::ROWB);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          sc[kbk][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][dc], sc[kbk][qb], 0, 0, 0);
      }
    // Issue order: each later K operand read two MFMA groups ahead of its use.
#pragma unroll
    for (int i = 0; i < 2 * C::DC - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, kQB, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kQB, 1);
  }

  // keys >= kv of a tile: element r of key block kbk is key 16kbk + 4g + r
  __device__ __forceinline__ void mask_tail(f32x4_t (&sc)[2][kQB], int kv) {
    if (__builtin_expect(kv < C::BN, 0)) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
        const int thr = kv - 16 * kbk - 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r >= thr)
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) sc[kbk][qb][r] = -INFINITY;
      }
    }
  }
  // A wave whose rows cross the frame boundary, on a key frame only one of
  // the two frames attends: removes the tile from the rows of the other
  // frame (bit qb of t1bits: this lane's row of block qb lies in the second
  // frame; keep_t1: the tile belongs to the second frame's rows).
  __device__ __forceinline__ void mask_lanes(f32x4_t (&sc)[2][kQB], int t1bits, bool keep_t1) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const bool in_t1 = (t1bits >> qb) & 1;
      const bool ok = in_t1 == keep_t1;
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[kbk][qb][r] = ok ? sc[kbk][qb][r] : -INFINITY;
    }
  }
  // The running max of each query block, raised lazily as in Block::fold_max.
  // Whether any row's tile max exceeds its reference by more than kMaxLag is
  // decided on each lane's part of the row (the scaled maximum is the maximum
  // of the scaled parts), so the reduction over the row's four lanes runs
  // only when a rescale follows.
  __device__ __forceinline__ void fold_max(const f32x4_t (&sc)[2][kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float mx = sc[0][qb][0];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kbk][qb][r]);
      if (__builtin_amdgcn_ballot_w64(mx * scale_log2 > m_run[qb] + kMaxLag) != 0) {
        const float mt = row4_max(mx) * scale_log2;
        const float m_new = fmaxf(m_run[qb], mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
#pragma unroll
        for (int r = 0; r < 4; ++r) lsum[qb][r] *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[qb][db][r] *= alpha;
        m_run[qb] = m_new;
      }
    }
  }
  // Probabilities, rounded to bf16, as the B operands of P·V (k-slot
  // 8g + 4kbk + r is key 16kbk + 4g + r).
  template <bool FIXED>
  __device__ __forceinline__ void probs(const f32x4_t (&sc)[2][kQB], bf16x8_t (&pb)[kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float neg_m = -m_run[qb];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pb[qb][4 * kbk + r] = (__bf16)__builtin_amdgcn_exp2f(
              FIXED ? sc[kbk][qb][r] : __builtin_fmaf(sc[kbk][qb][r], scale_log2, neg_m));
    }
  }
  // Oᵀ += Vᵀ·P with the V tile in buffer VBUF: one pair of transposing
  // reads per dim block, shared by the three query blocks; then the row
  // sums of the rounded P (so the weights sum to one) on the matrix cores.
  template <int VBUF>
  __device__ __forceinline__ void pv(const bf16x8_t (&pb)[kQB]) {
    const char *Vb = bufp(VBUF) + kTileOffV;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(Vb + vro[db]));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(Vb + vro[db] + 16 * C::ROWB));
      const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        oacc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[qb], oacc[qb][db], 0, 0, 0);
    }
    // Issue order: the reads of two dim blocks, then each block's three
    // MFMAs followed by the next block's reads (measured 4-5% faster than
    // the compiler's own order, with the K-read order of qk 2-3% more).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
#pragma unroll
    for (int i = 0; i < C::DB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, kQB, 2);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kQB, 2);
    bf16x8_t ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qb], lsum[qb], 0, 0, 0);
  }
  // One key tile from LDS buffer BUF.
  template <int BUF, bool FIXED>
  __device__ __forceinline__ void tile(int kv, bool lane_mask, int t1bits, bool keep_t1, const bf16x8_t (&kp)[2]) {
    f32x4_t sc[2][kQB];
    bf16x8_t pb[kQB];
    qk<BUF, FIXED>(sc, kp);
    mask_tail(sc, kv);
    if (__builtin_expect(lane_mask, 0)) mask_lanes(sc, t1bits, keep_t1);
    if constexpr (!FIXED) fold_max(sc);
    probs<FIXED>(sc, pb);
    pv<BUF>(pb);
  }
};

// The span kernel: one work item of kSpanRows consecutive query tokens per
// workgroup (see the top of the file).
template <int D>
__global__ __launch_bounds__(SpanCfg<D>::NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void lvsa_attn_span(Args a) {
  using C = SpanCfg<D>;
  __shared__ __attribute__((aligned(1024))) char lds0[C::LDS_BYTES / 2];  // K0 V0
  __shared__ __attribute__((aligned(1024))) char lds1[C::LDS_BYTES / 2];  // K1 V1
  SpanBlock<D> blk;
  blk.lds0 = lds0;
  blk.lds1 = lds1;
  const int tid = threadIdx.x;
  blk.lane = tid & 63;
  blk.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  blk.s16 = blk.lane & 15;
  blk.g = blk.lane >> 4;
  blk.scale_log2 = a.scale_log2;

  int item, half, slot;
  if (!take_item(a, reinterpret_cast<int *>(lds1), &item, &half, &slot)) return;
  const Item wi = decode_item<C::BM, true>(a, item);
  const int P = a.P;
  const u16 *kbase = a.k + (int64_t)wi.b * a.k_sb + (int64_t)wi.h * a.k_sh;
  const u16 *vbase = a.v + (int64_t)wi.b * a.v_sb + (int64_t)wi.h * a.v_sh;

  // ---- Q rows: the wave's 48 rows × D as B operands (rows past the item's
  // end read as zeros and are never stored)
  const int row0 = wi.tok0 + blk.wave * 16 * kQB;  // token of the wave's first row
  {
    const u16 *qh = a.q + (int64_t)wi.b * a.q_sb + (int64_t)wi.h * a.q_sh;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int row = row0 + 16 * qb + blk.s16;
      const bool ok = row < wi.tok_end;
      const u16 *qp = qh + (int64_t)(ok ? row : 0) * a.q_sn + blk.g * 8;
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) {
        bf16x8_t x = *reinterpret_cast<const bf16x8_t *>(qp + dc * 32);
        if (!ok) x = bf16x8_t{};
        blk.qf[qb][dc] = x;
      }
    }
  }
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) blk.oacc[qb][db] = f32x4_t{};
    blk.m_run[qb] = -FLT_MAX;
    blk.lsum[qb] = f32x4_t{};
  }
  blk.init_offsets(a.k_sn, a.v_sn);
  // Whether the wave has rows in the item (the last item of the sequence may
  // not fill every wave); which of the walk's frame memberships its rows need
  // (bit 0: rows in t0, bit 1: rows in t1); and, per lane, which of its
  // three rows lie in t1.
  const int compute = __builtin_amdgcn_readfirstlane(row0 < wi.tok_end ? 1 : 0);
  const bool two = wi.t1 != wi.t0;
  int need = 3;
  int t1bits = 0;
  if (two && compute) {
    const int f_first = row0 / P;
    const int f_last = min(row0 + 16 * kQB - 1, wi.tok_end - 1) / P;
    need = f_first == f_last ? (f_first == wi.t0 ? 1 : 2) : 3;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) t1bits |= ((row0 + 16 * qb + blk.s16) / P == wi.t1 ? 1 : 0) << qb;
  }
  need = __builtin_amdgcn_readfirstlane(need);

  // ---- the key walk: the union of the rows of t0 and t1
  SegIter it = make_walk(a, wi, half);
  const int n_walk = walk_tiles(it, C::BN);

  // ---- softmax reference, as in the frame kernel, per query row
  bool fixed = false;
  if (a.knorm) {
    const float kn = walk_key_norm(a, wi);
    float r_ref[kQB];
    bool all_ok = true;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float ss = 0.f;
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)(__bf16)((float)blk.qf[qb][dc][e] * a.scale_log2);
          ss = __builtin_fmaf(x, x, ss);
        }
      ss = row4_sum(ss);  // the four lane groups hold a quarter of the row each
      r_ref[qb] = __builtin_sqrtf(ss) * kn * (1.0f + 1.0f / 256.0f);
      all_ok = all_ok && (2.0f * r_ref[qb] <= kMaxRefGap);
    }
    fixed = __builtin_amdgcn_ballot_w64(!all_ok) == 0;
    if (fixed) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        blk.m_run[qb] = r_ref[qb];
#pragma unroll
        for (int r = 0; r < 4; ++r) blk.bias[qb][r] = -r_ref[qb];
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
          for (int e = 0; e < 8; ++e) blk.qf[qb][dc][e] = (__bf16)((float)blk.qf[qb][dc][e] * a.scale_log2);
      }
    }
  }

  // ---- main loop over key tiles, as in the frame kernel.  A tile is
  // computed by the waves whose rows attend its frame (every wave, unless
  // the item's rows cross a frame boundary).
  int pos = 0, kv = 0, mem = 0;
  auto advance = [&]() {  // next tile, moving to the next segment when needed
    pos += C::BN;
    if (__builtin_expect(pos >= it.ke, 0)) {
      it.next();
      pos = it.ks;
    }
    kv = min(C::BN, it.ke - pos);
    mem = it.mem;
  };
  auto issue = [&](int buf) {
    blk.template issue<false>(buf, kbase, a.k_sn, pos, kv);
    blk.template issue<true>(buf, vbase, a.v_sn, pos, kv);
  };
  if (n_walk > 0) {
    it.next();
    pos = it.ks;
    kv = min(C::BN, it.ke - pos);
    mem = it.mem;
    issue(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  auto run = [&](auto fixed_c) {
    constexpr bool F = decltype(fixed_c)::value;
    auto step = [&](auto buf_c, int kvj, int memj, const bf16x8_t (&kp)[2]) {
      constexpr int BUF = decltype(buf_c)::value;
      if (__builtin_expect(compute && (memj & need), 1)) {
        // a boundary-crossing wave, on a frame only one of its two frames attends
        const bool lm = need == 3 && memj != 3;
        blk.template tile<BUF, F>(kvj, lm, t1bits, memj == 2, kp);
      }
    };
    bf16x8_t kp[2];
    for (int i = 0; i + 1 < n_walk; i += 2) {
      const int kv0 = kv, mem0 = mem;
      blk.template kpre<0>(kp);
      advance();  // tile i+1 -> buffer 1
      issue(1);
      step(std::integral_constant<int, 0>{}, kv0, mem0, kp);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int kv1 = kv, mem1 = mem;
      blk.template kpre<1>(kp);
      if (i + 2 < n_walk) {  // tile i+2 -> buffer 0
        advance();
        issue(0);
      }
      step(std::integral_constant<int, 1>{}, kv1, mem1, kp);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if (n_walk & 1) {
      blk.template kpre<0>(kp);
      step(std::integral_constant<int, 0>{}, kv, mem, kp);
    }
  };
  if (fixed)
    run(std::true_type{});
  else
    run(std::false_type{});

  // ---- a half writes its partial record (Oᵀ accumulators; row sums and
  // references of the three blocks) for lvsa_combine_span
  if (half >= 0) {
    if (compute) {
      constexpr int R4 = kSpanPartialFloats(D) / 4;
      float4 *rec = reinterpret_cast<float4 *>(a.partial) +
                    ((int64_t)(slot * 2 + half) * C::NW + blk.wave) * R4 * 64 + blk.lane;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const f32x4_t o = blk.oacc[qb][db];
          rec[(qb * C::DB + db) * 64] = make_float4(o[0], o[1], o[2], o[3]);
        }
      // row sums: the combine kernel adds the four lanes of a row, so lanes
      // g > 0 contribute zero
      float l4[kQB];
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) l4[qb] = blk.g == 0 ? blk.lsum[qb][0] : 0.f;
      rec[(kQB * C::DB) * 64] = make_float4(l4[0], l4[1], l4[2], blk.m_run[0]);
      rec[(kQB * C::DB + 1) * 64] = make_float4(blk.m_run[1], blk.m_run[2], 0.f, 0.f);
    }
    return;
  }
  // ---- epilogue: normalise, round to bf16, store (each lane: 4 dims of
  // every 16-dim block of its three rows)
  {
    u16 *oh = a.o + (int64_t)wi.b * a.o_sb + (int64_t)wi.h * a.o_sh;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float l_tot = blk.lsum[qb][0];
      const int row = row0 + 16 * qb + blk.s16;
      if (row < wi.tok_end) {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        u16 *op = oh + (int64_t)row * a.o_sn + 4 * blk.g;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          bf16x4_t o4;
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = (__bf16)(blk.oacc[qb][db][r] * inv);
          *reinterpret_cast<bf16x4_t *>(op + 16 * db) = o4;
        }
      }
    }
  }
}

// Merges the two halves of every split item of the span kernel: one
// workgroup per record slot, one wave per 48 query rows as in
// lvsa_attn_span (the frame kernel's merge, per query block).
template <int D>
__global__ __launch_bounds__(SpanCfg<D>::NW * 64) void lvsa_combine_span(Args a) {
  using C = SpanCfg<D>;
  const int x = blockIdx.x / a.split_cap, j = blockIdx.x % a.split_cap;
  int base, cnt;
  xcd_range(a.n_wg, x, &base, &cnt);
  const int S = split_count(a.split_cap, cnt);
  if (j >= S) return;
  const Item wi = decode_item<C::BM, true>(a, base + (cnt - S) + j);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s16 = lane & 15, g = lane >> 4;
  const int row0 = wi.tok0 + wave * 16 * kQB;
  if (row0 >= wi.tok_end) return;
  constexpr int R4 = kSpanPartialFloats(D) / 4;
  const float4 *r0 = reinterpret_cast<const float4 *>(a.partial) + ((int64_t)(blockIdx.x * 2) * C::NW + wave) * R4 * 64 + lane;
  const float4 *r1 = r0 + (int64_t)C::NW * R4 * 64;
  const float4 a0 = r0[(kQB * C::DB) * 64], a1 = r1[(kQB * C::DB) * 64];
  const float4 b0 = r0[(kQB * C::DB + 1) * 64], b1 = r1[(kQB * C::DB + 1) * 64];
  const float l0[kQB] = {a0.x, a0.y, a0.z}, l1[kQB] = {a1.x, a1.y, a1.z};
  const float m0[kQB] = {a0.w, b0.x, b0.y}, m1[kQB] = {a1.w, b1.x, b1.y};
  u16 *oh = a.o + (int64_t)wi.b * a.o_sb + (int64_t)wi.h * a.o_sh;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float m = fmaxf(m0[qb], m1[qb]);
    const float w0 = __builtin_amdgcn_exp2f(m0[qb] - m);
    const float w1 = __builtin_amdgcn_exp2f(m1[qb] - m);
    const float l_tot = row4_sum(w0 * l0[qb] + w1 * l1[qb]);
    const int row = row0 + 16 * qb + s16;
    if (row >= wi.tok_end) continue;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    u16 *op = oh + (int64_t)row * a.o_sn + 4 * g;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const float4 o0 = r0[(qb * C::DB + db) * 64], o1 = r1[(qb * C::DB + db) * 64];
      bf16x4_t o4;
      o4[0] = (__bf16)((w0 * o0.x + w1 * o1.x) * inv);
      o4[1] = (__bf16)((w0 * o0.y + w1 * o1.y) * inv);
      o4[2] = (__bf16)((w0 * o0.z + w1 * o1.z) * inv);
      o4[3] = (__bf16)((w0 * o0.w + w1 * o1.w) * inv);
      *reinterpret_cast<bf16x4_t *>(op + 16 * db) = o4;
    }
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

// Device address of `scratch` on each device, taken once per device with
// that device current.
struct ScratchAddr {
  std::once_flag once[64];
  void *ptr[64] = {};
  hipError_t err[64] = {};
};
ScratchAddr g_scratch;

int static_scratch_ptr(int dev, void **out) {
  std::call_once(g_scratch.once[dev], [dev]() {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch.err[dev] = e;
    g_scratch.ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  if (g_scratch.err[dev] != hipSuccess || !g_scratch.ptr[dev])
    return lvsa::fail(LVSA_ERR_HIP, "device %d: no address for the static scratch (%s)", dev,
                      hipGetErrorString(g_scratch.err[dev]));
  *out = g_scratch.ptr[dev];
  return LVSA_OK;
}

int check_tensor(const lvsa_tensor *x, const char *name) {
  if (!x || !x->data) return lvsa::fail(LVSA_ERR_ARG, "%s: NULL tensor or data pointer", name);
  if (x->dtype != LVSA_DTYPE_BF16) return lvsa::fail(LVSA_ERR_DTYPE, "%s: dtype %d, only bf16 is supported", name, x->dtype);
  if (x->B < 1 || x->H < 1 || x->N < 1) return lvsa::fail(LVSA_ERR_SHAPE, "%s: empty or negative B/H/N", name);
  if (x->B > INT32_MAX || x->H > INT32_MAX || x->N > INT32_MAX)
    return lvsa::fail(LVSA_ERR_SHAPE, "%s: B/H/N above 2^31", name);
  if (x->D != 64 && x->D != 128) return lvsa::fail(LVSA_ERR_SHAPE, "%s: D=%lld, supported 64 and 128", name, (long long)x->D);
  if (reinterpret_cast<uintptr_t>(x->data) % 16) return lvsa::fail(LVSA_ERR_SHAPE, "%s: data not 16-byte aligned", name);
  if (x->stride_n < x->D || x->stride_b < 0 || x->stride_h < 0 || x->stride_n % 8 || x->stride_h % 8 || x->stride_b % 8)
    return lvsa::fail(LVSA_ERR_SHAPE, "%s: strides must be multiples of 8 elements with stride_n >= D", name);
  if (x->stride_n > (int64_t{1} << 24))
    return lvsa::fail(LVSA_ERR_SHAPE, "%s: stride_n above 2^24 elements is not supported", name);
  // byte extent, in floating point first so that the int64 arithmetic below
  // and in extent() cannot overflow
  const double span = (double)(x->B - 1) * (double)x->stride_b + (double)(x->H - 1) * (double)x->stride_h +
                      (double)(x->N - 1) * (double)x->stride_n + (double)x->D;
  if (span * 2.0 > 0x1p62) return lvsa::fail(LVSA_ERR_SHAPE, "%s: strides span more than 2^62 bytes", name);
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

// Launches, on one stream: the key-norm pass (with a workspace), the
// attention kernel ATTN (NT threads per workgroup) and the merge of split
// items MERGE.
template <int D, void (*ATTN)(Args), void (*MERGE)(Args), int NT>
int launch(const Args &args, int n_frames, hipStream_t stream) {
  if (args.knorm) {
    hipLaunchKernelGGL((lvsa_key_norms<D>), dim3(n_frames), dim3(256), 0, stream, args.k, args.k_sb, args.k_sh,
                       args.k_sn, args.H, args.T, args.P, const_cast<float *>(args.knorm), args.tickets);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return lvsa::fail(LVSA_ERR_HIP, "key-norm kernel launch failed: %s", hipGetErrorString(e));
  }
  // With tickets: one workgroup per ticket (items, plus one more per split
  // item), and 1/8 more, so that the fastest XCD can take over up to that
  // share of the others' items.
  const int64_t grid =
      args.tickets ? args.n_wg + (int64_t)kNumXcd * args.split_cap + args.n_wg / 8 + kNumXcd : args.n_wg;
  hipLaunchKernelGGL(ATTN, dim3((unsigned)grid), dim3(NT), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return lvsa::fail(LVSA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  if (args.tickets && args.split_cap > 0) {
    hipLaunchKernelGGL(MERGE, dim3(kNumXcd * args.split_cap), dim3(NT), 0, stream, args);
    e = hipGetLastError();
    if (e != hipSuccess) return lvsa::fail(LVSA_ERR_HIP, "combine kernel launch failed: %s", hipGetErrorString(e));
  }
  return lvsa::ok();
}
template <int D>
int launch_frame(const Args &args, int n_frames, hipStream_t stream) {
  return launch<D, lvsa_attn_frame<D>, lvsa_combine_frame<D>, kFrameWaves * 64>(args, n_frames, stream);
}
template <int D>
int launch_span(const Args &args, int n_frames, hipStream_t stream) {
  return launch<D, lvsa_attn_span<D>, lvsa_combine_span<D>, SpanCfg<D>::NW * 64>(args, n_frames, stream);
}

// How a call is cut into work items.  Frames of at least kSpanRows tokens
// (every video workload): items of kSpanRows consecutive tokens, which may
// cross one frame boundary, for 8-wave workgroups of the span kernel (one
// per CU).  Shorter frames: items of 128 rows of one frame for 4-wave
// workgroups of the frame kernel.
struct Plan {
  bool span;
  int nw, q_tiles;
  int64_t items;
  int32_t split_per_xcd;  // items per XCD range run as two halves, at most
};
Plan plan_for(int64_t B, int64_t H, int64_t N, int64_t T) {
  Plan p;
  const int64_t P = N / T;
  p.span = P >= kSpanRows;
  if (p.span) {
    p.nw = SpanCfg<128>::NW;
    p.q_tiles = (int)((N + kSpanRows - 1) / kSpanRows);
    p.items = B * H * p.q_tiles;
    p.split_per_xcd = 32;
  } else {
    p.nw = kFrameWaves;
    p.q_tiles = (int)((P + kFrameWaves * 32 - 1) / (kFrameWaves * 32));
    p.items = B * H * T * p.q_tiles;
    p.split_per_xcd = 96;
  }
  return p;
}

// Workspace: the key-norm table (B·H·T floats), then, at the next
// 256-byte boundary, the 8 ticket counters (256 bytes), then the partial
// records of the split items (8·split_cap slots × 2 halves × NW waves × 64
// lanes × kSpanPartialFloats(D) or kPartialFloats(D) floats).
int64_t norms_bytes_for(int64_t B, int64_t H, int64_t T) {
  return ((B * H * T * (int64_t)sizeof(float) + 255) / 256) * 256;
}
// At most a quarter of every XCD range is split.
int32_t split_cap_for(const Plan &p) {
  return (int32_t)std::min<int64_t>(p.split_per_xcd, p.items / (4 * kNumXcd));
}
// Bytes of partial records per unit of split_cap (one slot per XCD).
int64_t split_unit_bytes(const Plan &p, int64_t D) {
  if (p.span) return (int64_t)kNumXcd * 2 * p.nw * 64 * kSpanPartialFloats((int)D) * 4;
  return (int64_t)kNumXcd * 2 * p.nw * 64 * kPartialFloats((int)D) * 4;
}
int64_t workspace_bytes_for(int64_t B, int64_t H, int64_t N, int64_t D, int64_t T, int32_t split_cap) {
  return norms_bytes_for(B, H, T) + 256 + split_cap * split_unit_bytes(plan_for(B, H, N, T), D);
}
int64_t workspace_bytes_for(int64_t B, int64_t H, int64_t N, int64_t D, int64_t T) {
  return workspace_bytes_for(B, H, N, D, T, split_cap_for(plan_for(B, H, N, T)));
}

int attention_impl(const lvsa_tensor *q, const lvsa_tensor *k, const lvsa_tensor *v,
                   const int32_t *row_ptr_dev, const int32_t *col_idx_dev, int32_t T, int32_t nnz,
                   lvsa_tensor *out, float scale, void *workspace, int64_t workspace_bytes, bool use_ws,
                   void *stream, int32_t split_cap_limit = -1) {
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
  if ((double)q->B * (double)q->H * (double)q->N > 0x1p46)
    return lvsa::fail(LVSA_ERR_SHAPE, "B*H*N = %.3g tokens too large", (double)q->B * (double)q->H * (double)q->N);
  if (!row_ptr_dev || !col_idx_dev || nnz < 0)
    return lvsa::fail(LVSA_ERR_ARG, "row_ptr/col_idx NULL or nnz < 0");
  {
    uint32_t bits;  // exponent all ones: inf or NaN (a bit test no fast-math flag can fold)
    std::memcpy(&bits, &scale, sizeof bits);
    if ((bits & 0x7f800000u) == 0x7f800000u) return lvsa::fail(LVSA_ERR_ARG, "scale is not finite");
  }
  int32_t split_cap = 0;
  if (use_ws) {
    split_cap = split_cap_for(plan_for(q->B, q->H, q->N, T));
    if (split_cap_limit >= 0) split_cap = std::min(split_cap, split_cap_limit);
    const int64_t need = workspace_bytes_for(q->B, q->H, q->N, q->D, T, split_cap);
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
  const Plan plan = plan_for(q->B, q->H, q->N, T);
  const int q_tiles = plan.q_tiles;
  const int64_t n_wg = plan.items;
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
  a.split_cap = split_cap;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n_frames = (int)(q->B * q->H * T);
  if (plan.span) {
    if (D == 128) return launch_span<128>(a, n_frames, s);
    return launch_span<64>(a, n_frames, s);
  }
  if (D == 128) return launch_frame<128>(a, n_frames, s);
  return launch_frame<64>(a, n_frames, s);
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
  if (N > INT32_MAX / 2 || (double)B * (double)H * (double)N > 0x1p40)
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

extern "C" int lvsa_attention_ws_static(const lvsa_tensor *q, const lvsa_tensor *k, const lvsa_tensor *v,
                                        const int32_t *row_ptr_dev, const int32_t *col_idx_dev,
                                        int32_t T, int32_t nnz, lvsa_tensor *out, float scale, void *stream) {
  int rc, dev;
  if ((rc = check_tensor(q, "q"))) return rc;
  if (T < 1) return lvsa::fail(LVSA_ERR_ARG, "T=%d: need T >= 1", T);
  if (q->N % T) return lvsa::fail(LVSA_ERR_SHAPE, "N=%lld is not a multiple of T=%d", (long long)q->N, T);
  // The key-norm table (one float per (b, h, frame)) and the counters must
  // fit; the split items take what is left (fewer items than
  // lvsa_attention_ws splits, when the room is smaller).
  const double frames = (double)q->B * (double)q->H * (double)T;
  if (frames * 4.0 + 512.0 > (double)kStaticScratchBytes)
    return lvsa::fail(LVSA_ERR_CAPACITY,
                      "B*H*T = %.0f (b, h, frame) entries do not fit the static scratch of %lld bytes (at most "
                      "%lld); use lvsa_attention_ws with a caller workspace",
                      frames, (long long)kStaticScratchBytes, (long long)((kStaticScratchBytes - 512) / 4));
  if ((rc = check_device(&dev))) return rc;
  void *ws;
  if ((rc = static_scratch_ptr(dev, &ws))) return rc;
  const int64_t fixed = norms_bytes_for(q->B, q->H, T) + 256;
  const int32_t cap = (int32_t)std::min<int64_t>(
      INT32_MAX, (kStaticScratchBytes - fixed) / split_unit_bytes(plan_for(q->B, q->H, q->N, T), q->D));
  return attention_impl(q, k, v, row_ptr_dev, col_idx_dev, T, nnz, out, scale, ws, kStaticScratchBytes, true,
                        stream, cap);
}
