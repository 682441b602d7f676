// zero_kernels.hip -- gfx950 kernels of the ZeRO shard step.
//
// Two kernel families, both bound by HBM bandwidth and written for CDNA4's
// 64-lane wavefronts (no MFMA: nothing here is a contraction):
//
//  * step kernels: for each element of the owner's shard, fold the N_d ranks'
//    16-bit gradient contributions in fixed rank order in fp32 (the
//    arithmetic of reduce-scatter), then run the mixed-precision Adam update on
//    the fp32 master weight and moments and store the rounded 16-bit parameter
//    into the all-gather buffer -- all in registers, one HBM pass.  In the
//    vector kernel each lane owns two groups of 4 elements laid out so that
//    every wave-wide load or store covers whole contiguous 128-byte lines:
//    per rank two 8-byte loads, per fp32 state array two 16-byte loads and
//    stores, two 8-byte parameter stores.  Every rank pointer and segment
//    offset is wave-uniform, so address arithmetic stays on the scalar unit
//    and vector accesses are an SGPR base plus a 32-bit lane offset.  Stores
//    can be held back to a device-wide write window (see await_write_window).
//
//  * copy kernel: destination-aligned 16-byte copies used by flatten (ragged
//    tensors into padded buckets, at any element offset) and gather_pack
//    (shards into the full buffer).  A misaligned source is realigned in
//    registers with byte funnel shifts; partial units at the ends of an entry
//    are copied element by element, so no byte outside an entry is touched.
//    Interior workgroups issue all of a lane's loads before its stores.
//
// Floating point: compiled with -ffp-contract=off; fp32 division and square
// root are HIP's correctly rounded defaults; denormals are preserved.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "zero_internal.h"

#pragma clang fp contract(off)

namespace zk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Global-address-space views, so that accesses are global_* (not flat_*).
typedef __attribute__((address_space(1))) u32x4 gu32x4;
typedef __attribute__((address_space(1))) f32x4 gf32x4;
typedef __attribute__((address_space(1))) u32x2 gu32x2;
typedef __attribute__((address_space(1))) uint16_t gu16;
typedef __attribute__((address_space(1))) uint32_t gu32;
typedef __attribute__((address_space(1))) float gf32;

template <typename T>
__device__ __forceinline__ T gaddr(const void* p) {
  return (T)p;
}
template <typename T>
__device__ __forceinline__ T gaddr(uint64_t p) {
  return (T)(uintptr_t)p;
}

// Streaming (non-temporal) accesses: every byte of the step is touched once.
__device__ __forceinline__ u32x4 ld_nt(const gu32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ f32x4 ld_nt(const gf32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2 ld_nt(const gu32x2* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(gu32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt(gu32x2* p, u32x2 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt(gf32x4* p, f32x4 v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int GDT>
__device__ __forceinline__ float widen1(uint32_t h) {
  if constexpr (GDT == ZERO_BF16) return __uint_as_float(h << 16);
  else return f16_bits_to_f32(h);
}

// fp32 -> 16-bit, round to nearest even (gfx950 conversion instructions).
template <int PDT>
__device__ __forceinline__ uint32_t narrow1(float x) {
  if constexpr (PDT == ZERO_BF16) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

struct AdamC {
  float b1, c1, b2, c2, bc1, bc2, lr, eps, gs;
};

__device__ __forceinline__ AdamC load_consts(const StepArgs& a) {
  return AdamC{a.c[0], a.c[1], a.c[2], a.c[3], a.c[4], a.c[5], a.c[6], a.c[7], a.c[8]};
}

// Textbook Adam on one element (bias-corrected moments, eps outside the
// square root, no weight decay).  One fp32 operation per statement.
__device__ __forceinline__ void adam1(const AdamC& k, float g, float& w, float& m, float& v) {
  const float m_old = k.b1 * m;
  const float m_in = k.c1 * g;
  m = m_old + m_in;
  const float g2 = g * g;
  const float v_old = k.b2 * v;
  const float v_in = k.c2 * g2;
  v = v_old + v_in;
  const float mh = m / k.bc1;
  const float vh = v / k.bc2;
  const float root = __builtin_sqrtf(vh);
  const float den = root + k.eps;
  const float upd = mh / den;
  const float delta = k.lr * upd;
  w = w - delta;
}

// Keeps the eight values computed before this point: the compiler may not
// sink their arithmetic (and with it the loads feeding it) below a following
// wait loop.
__device__ __forceinline__ void pin8(float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(x[i]));
}

// Write window.  With period > 0, a wave whose results are ready stores them
// only while the device's real-time counter is within the first `open` ticks
// of a `period`-tick period; otherwise it sleeps until the next period begins.
// The counter is read on the scalar unit, so the branch is wave-uniform.  The
// wait ends when the counter reaches the target or after kWindowSpinMax
// iterations, whichever comes first.
//
// Why: the step reads ~10 bytes for every byte it writes.  When each wave
// stores as soon as it is done, writes reach HBM as a thin stream interleaved
// with the reads, and every read/write turnaround of the DRAM costs far more
// than the written bytes themselves.  Gathering the stores of all waves into
// short bursts lets the memory controller drain them together.
__device__ __forceinline__ void await_write_window(uint32_t period, uint32_t open) {
  if (period == 0) return;
  const uint64_t now = __builtin_amdgcn_s_memrealtime();
  const uint64_t phase = now % period;
  if (phase < open) return;
  const uint64_t target = now - phase + period;
  for (uint32_t i = 0; i < kWindowSpinMax && __builtin_amdgcn_s_memrealtime() < target; ++i)
    __builtin_amdgcn_s_sleep(4);
}

// The store window's other half: a wave about to start its loads waits
// through the opening, so that while the device's stores drain the reads of
// newly started waves do not mix with them.  Waves already loading are not
// held (only the first load of a wave is gated).  Measured on MI355X against
// the store window alone: the 13B step (N_d = 16, 24% of its bytes written)
// 1.5% faster, N_d = 24 and 32 0.6-1.2%; the 7.5B step (9% written) about 1%
// faster in fresh processes and unchanged late in a long one; the reduction
// (3% written) unchanged.  Gating every rank batch as well helped N_d = 16 a
// little more but cost N_d = 24 and 32 up to 3%.
__device__ __forceinline__ void await_read_window(uint32_t period, uint32_t open) {
  if (period == 0 || open >= period) return;   // no window, or no closed phase to load in
  const uint64_t now = __builtin_amdgcn_s_memrealtime();
  const uint64_t phase = now % period;
  if (phase >= open) return;
  const uint64_t target = now - phase + open;
  for (uint32_t i = 0; i < kWindowSpinMax && __builtin_amdgcn_s_memrealtime() < target; ++i)
    __builtin_amdgcn_s_sleep(4);
}

// Segment handled by this workgroup (wave-uniform linear scan, <= 64 entries).
__device__ __forceinline__ int find_seg(const StepArgs& a, int blk) {
  int s = 0;
  for (int i = 1; i < a.n_seg; ++i)
    if (a.seg[i].block_start <= blk) s = i;
  return s;
}

// Byte address of rank q's contribution at the segment's first element.
__device__ __forceinline__ uint64_t rank_base(const StepArgs& a, int q, int64_t shard_off,
                                              int64_t full_off) {
  const bool full = (a.full_mask[q >> 5] >> (q & 31)) & 1u;
  return (uint64_t)(uintptr_t)a.grad[q] + (uint64_t)((full ? full_off : shard_off) * 2);
}

// Lane -> element mapping of the vector kernel.  A wave owns a tile of 512
// consecutive elements; lane l owns two groups of 4: elements [4l, 4l+4) and
// [256+4l, 256+4l+4) of the tile.  Every memory instruction of the wave then
// covers one contiguous span -- 512 bytes of a 16-bit array, 1 KiB of an fp32
// array -- made of whole 128-byte lines, so no line is fetched or written
// back in halves by two different instructions.
constexpr uint32_t kTile = 512;
constexpr uint32_t kHalf = 256;

__device__ __forceinline__ const gu32x2* grad_pair(const StepArgs& a, int q, int64_t shard_off,
                                                   int64_t full_off, uint32_t boff) {
  return gaddr<const gu32x2*>(rank_base(a, q, shard_off, full_off)) + (boff >> 3);
}

// 4 packed 16-bit values -> 4 fp32 values (exact widening).
template <int GDT>
__device__ __forceinline__ void widen4(const u32x2 r, float* x) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if constexpr (GDT == ZERO_BF16) {
      x[2 * i] = __uint_as_float(r[i] << 16);
      x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    } else {
      x[2 * i] = f16_bits_to_f32(r[i] & 0xffffu);
      x[2 * i + 1] = f16_bits_to_f32(r[i] >> 16);
    }
  }
}

// Ends a batch of the fold: the batch's adds complete before this point and
// no later load is hoisted above it (the "memory" clobber), so a wave holds
// one batch of loaded ranks in registers at a time.  Without it the compiler
// hoists the loads of the whole unrolled rank loop (108 VGPRs for the bf16
// reduce-only kernel, 172 for fp16), halving or quartering occupancy.
__device__ __forceinline__ void end_batch(float (&acc)[8]) {
  asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
               "+v"(acc[6]), "+v"(acc[7])::"memory");
}

// Fold the launch's ranks for the lane's two 4-element groups (byte offsets
// boa, bob of each rank's segment base).  acc[0..3] is group a, acc[4..7]
// group b.  CONT = false: the fold starts from the first rank's value;
// CONT = true: every rank is added to the incoming acc (continuing a fold
// begun by an earlier launch).  Loads are issued in batches of B ranks ahead
// of their adds, so B KiB per wave are in flight; adds keep rank order.  fp16
// batches are 8 ranks: widening fp16 takes more registers than bf16's shifts,
// and 16 would cost occupancy.
template <int GDT, int NDC, bool CONT>
__device__ __forceinline__ void fold(const StepArgs& a, int64_t shard_off, int64_t full_off,
                                     uint32_t boa, uint32_t bob, float (&acc)[8]) {
  auto take = [&](const u32x2 ra, const u32x2 rb, bool first) {
    float x[8];
    widen4<GDT>(ra, x);
    widen4<GDT>(rb, x + 4);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = first ? x[k] : acc[k] + x[k];
  };
  if constexpr (NDC > 0) {
    constexpr int B = NDC < 16 ? NDC : (GDT == ZERO_F16 ? 8 : 16);
#pragma unroll
    for (int q0 = 0; q0 < NDC; q0 += B) {
      u32x2 ra[B], rb[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        ra[i] = ld_nt(grad_pair(a, q0 + i, shard_off, full_off, boa));
        rb[i] = ld_nt(grad_pair(a, q0 + i, shard_off, full_off, bob));
      }
#pragma unroll
      for (int i = 0; i < B; ++i) take(ra[i], rb[i], !CONT && q0 + i == 0);
      end_batch(acc);
    }
  } else {
    const int n = a.n_ranks;
    int q = 0;
    if (!CONT) {
      take(ld_nt(grad_pair(a, 0, shard_off, full_off, boa)),
           ld_nt(grad_pair(a, 0, shard_off, full_off, bob)), true);
      q = 1;
    }
    constexpr int B = 8;
    for (; q + B <= n; q += B) {
      u32x2 ra[B], rb[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        ra[i] = ld_nt(grad_pair(a, q + i, shard_off, full_off, boa));
        rb[i] = ld_nt(grad_pair(a, q + i, shard_off, full_off, bob));
      }
#pragma unroll
      for (int i = 0; i < B; ++i) take(ra[i], rb[i], false);
      end_batch(acc);
    }
    for (; q < n; ++q)
      take(ld_nt(grad_pair(a, q, shard_off, full_off, boa)),
           ld_nt(grad_pair(a, q, shard_off, full_off, bob)), false);
  }
}

// fp32 groups: x[0..3] at element ea, x[4..7] at element eb of array base p.
__device__ __forceinline__ void load_groups(const float* p, uint32_t ea, uint32_t eb, float (&x)[8]) {
  const f32x4 u = ld_nt(gaddr<const gf32x4*>(p) + (ea >> 2));
  const f32x4 w = ld_nt(gaddr<const gf32x4*>(p) + (eb >> 2));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[k] = u[k];
    x[4 + k] = w[k];
  }
}

__device__ __forceinline__ void store_groups(float* p, uint32_t ea, uint32_t eb, bool vb,
                                             const float (&x)[8]) {
  st_nt(gaddr<gf32x4*>(p) + (ea >> 2), f32x4{x[0], x[1], x[2], x[3]});
  if (vb) st_nt(gaddr<gf32x4*>(p) + (eb >> 2), f32x4{x[4], x[5], x[6], x[7]});
}

// One element e of a segment, with the same arithmetic as the vector kernel:
// scalar loads at any element alignment.  The element kernel runs it for
// every element; the vector kernel for the last (< 4) elements of a segment
// whose length is not a multiple of 4.
template <int MODE, int GDT, int PDT>
__device__ __forceinline__ void step_one(const StepArgs& a, int64_t shard_off, int64_t full_off,
                                         int64_t dst_off, uint32_t e) {
  float g;
  if constexpr (MODE == kFromReduced) {
    g = gaddr<const gf32*>(a.reduced)[shard_off + e];
  } else {
    const int n = a.n_ranks;
    float acc;
    int q = 0;
    if (MODE == kReduceOnly && (a.flags & kFlagInitFromOut)) {
      acc = gaddr<const gf32*>(a.out)[shard_off + e];
    } else {
      acc = widen1<GDT>(gaddr<const gu16*>(rank_base(a, 0, shard_off, full_off))[e]);
      q = 1;
    }
    for (; q < n; ++q)
      acc = acc + widen1<GDT>(gaddr<const gu16*>(rank_base(a, q, shard_off, full_off))[e]);
    if (MODE == kReduceOnly) {
      if (a.flags & kFlagApplyScale) acc = acc * a.c[8];
      gaddr<gf32*>(a.out)[shard_off + e] = acc;
      return;
    }
    g = acc * a.c[8];
  }
  if constexpr (MODE != kReduceOnly) {
    const AdamC k = load_consts(a);
    gf32* wp = gaddr<gf32*>(a.master);
    gf32* mp = gaddr<gf32*>(a.m);
    gf32* vp = gaddr<gf32*>(a.v);
    float w = wp[shard_off + e], m = mp[shard_off + e], v = vp[shard_off + e];
    adam1(k, g, w, m, v);
    wp[shard_off + e] = w;
    mp[shard_off + e] = m;
    vp[shard_off + e] = v;
    gaddr<gu16*>(a.dst)[dst_off + e] = (uint16_t)narrow1<PDT>(w);
  }
}

// Element kernel: one element per lane, any element alignment (taken for
// pieces whose offsets are not multiples of 4 elements, or when a base
// address is not 16-byte aligned).
template <int MODE, int GDT, int PDT>
__global__ void __launch_bounds__(kThreads) step_elem_kernel(const StepArgs a) {
  const int blk = blockIdx.x;
  const int s = find_seg(a, blk);
  const uint32_t len = (uint32_t)a.seg[s].len;
  const uint32_t e = (uint32_t)(blk - a.seg[s].block_start) * kThreads + threadIdx.x;
  if (e >= len) return;
  step_one<MODE, GDT, PDT>(a, a.seg[s].shard_off, a.seg[s].full_off, a.seg[s].dst_off, e);
}

// Vector kernel.  The host takes it only when a segment's offsets (shard,
// full-buffer where a rank reads one, destination) are multiples of 4
// elements and every base address is 16-byte aligned; the length is free.  A
// segment's last wave tile may be partial: a lane whose second group lies
// past the end loads the first group's addresses again (in bounds) and skips
// those stores, and the last (< 4) elements of a length that is not a
// multiple of 4 go through the element routine.
template <int MODE, int GDT, int PDT, int NDC>
__global__ void __launch_bounds__(kStepThreads) step_vec_kernel(const StepArgs a) {
  const int blk = blockIdx.x;
  const int s = find_seg(a, blk);
  const int64_t shard_off = a.seg[s].shard_off;
  const int64_t full_off = a.seg[s].full_off;
  const int64_t dst_off = a.seg[s].dst_off;
  const uint32_t len = (uint32_t)a.seg[s].len;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t tile = (uint32_t)(blk - a.seg[s].block_start) * (kStepThreads * kStepVec) +
                        (threadIdx.x >> 6) * kTile;
  const uint32_t ea = tile + 4u * lane;
  if (ea >= len) return;
  if (ea + 4u > len) {   // the segment's partial last group
    for (uint32_t e = ea; e < len; ++e) step_one<MODE, GDT, PDT>(a, shard_off, full_off, dst_off, e);
    return;
  }
  const bool vb = ea + kHalf + 4u <= len;        // second group whole
  const bool tb = !vb && ea + kHalf < len;       // second group partial
  const uint32_t eb = vb ? ea + kHalf : ea;

  float g[8];
  if constexpr (MODE == kFromReduced) {
    // About one byte written per byte read, as in a copy: group by group (load
    // the lane's 4 elements of every array, update, store, then the next 4),
    // so a lane has 64 bytes of loads in flight rather than 128.  A plain
    // copy runs fastest at that depth on MI355X; here it is ~1% faster than
    // both groups at once, and the arithmetic is the same.
    const AdamC k = load_consts(a);
    gu32x2* const dp = gaddr<gu32x2*>((uint16_t*)a.dst + dst_off);
    auto group = [&](uint32_t e) {
      const f32x4 g4 = ld_nt(gaddr<const gf32x4*>(a.reduced + shard_off) + (e >> 2));
      const f32x4 w4 = ld_nt(gaddr<const gf32x4*>(a.master + shard_off) + (e >> 2));
      const f32x4 m4 = ld_nt(gaddr<const gf32x4*>(a.m + shard_off) + (e >> 2));
      const f32x4 v4 = ld_nt(gaddr<const gf32x4*>(a.v + shard_off) + (e >> 2));
      float w[4], m[4], v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = w4[i];
        m[i] = m4[i];
        v[i] = v4[i];
        adam1(k, g4[i], w[i], m[i], v[i]);
      }
      st_nt(gaddr<gf32x4*>(a.master + shard_off) + (e >> 2), f32x4{w[0], w[1], w[2], w[3]});
      st_nt(gaddr<gf32x4*>(a.m + shard_off) + (e >> 2), f32x4{m[0], m[1], m[2], m[3]});
      st_nt(gaddr<gf32x4*>(a.v + shard_off) + (e >> 2), f32x4{v[0], v[1], v[2], v[3]});
      st_nt(dp + (e >> 2), u32x2{narrow1<PDT>(w[0]) | (narrow1<PDT>(w[1]) << 16),
                                 narrow1<PDT>(w[2]) | (narrow1<PDT>(w[3]) << 16)});
    };
    group(ea);
    if (vb) group(eb);
    if (tb)
      for (uint32_t e = ea + kHalf; e < len; ++e) step_one<MODE, GDT, PDT>(a, shard_off, full_off, dst_off, e);
    return;
  } else if constexpr (MODE == kFused) {
    float acc[8];
    await_read_window(a.win_period, a.win_open);
    fold<GDT, NDC, false>(a, shard_off, full_off, ea * 2u, eb * 2u, acc);
    const float gs = a.c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] = acc[k] * gs;
  } else {  // kReduceOnly
    float acc[8];
    if (a.flags & kFlagInitFromOut) {
      // The fp32 prefix of the fold was stored exactly by the previous launch.
      load_groups(a.out + shard_off, ea, eb, acc);
      fold<GDT, NDC, true>(a, shard_off, full_off, ea * 2u, eb * 2u, acc);
    } else {
      await_read_window(a.win_period, a.win_open);
      fold<GDT, NDC, false>(a, shard_off, full_off, ea * 2u, eb * 2u, acc);
    }
    if (a.flags & kFlagApplyScale) {
      const float gs = a.c[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = acc[k] * gs;
    }
    pin8(acc);
    await_write_window(a.win_period, a.win_open);
    store_groups(a.out + shard_off, ea, eb, vb, acc);
  }

  if constexpr (MODE != kReduceOnly) {
    const AdamC k = load_consts(a);
    float w[8], m[8], v[8];
    load_groups(a.master + shard_off, ea, eb, w);
    load_groups(a.m + shard_off, ea, eb, m);
    load_groups(a.v + shard_off, ea, eb, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) adam1(k, g[i], w[i], m[i], v[i]);
    pin8(w);
    pin8(m);
    pin8(v);
    await_write_window(a.win_period, a.win_open);
    store_groups(a.master + shard_off, ea, eb, vb, w);
    store_groups(a.m + shard_off, ea, eb, vb, m);
    store_groups(a.v + shard_off, ea, eb, vb, v);
    const u32x2 pa = {narrow1<PDT>(w[0]) | (narrow1<PDT>(w[1]) << 16),
                      narrow1<PDT>(w[2]) | (narrow1<PDT>(w[3]) << 16)};
    const u32x2 pb = {narrow1<PDT>(w[4]) | (narrow1<PDT>(w[5]) << 16),
                      narrow1<PDT>(w[6]) | (narrow1<PDT>(w[7]) << 16)};
    gu32x2* const dp = gaddr<gu32x2*>((uint16_t*)a.dst + dst_off);
    st_nt(dp + (ea >> 2), pa);
    if (vb) st_nt(dp + (eb >> 2), pb);
  }
  if (tb)
    for (uint32_t e = ea + kHalf; e < len; ++e) step_one<MODE, GDT, PDT>(a, shard_off, full_off, dst_off, e);
}


// ---------------------------------------------------------------------------
// Copies (flatten, gather_pack)
// ---------------------------------------------------------------------------

__device__ __forceinline__ int find_ent(const CopyArgs& a, int blk) {
  int lo = 0, hi = a.n_ent - 1;   // last entry whose block_start <= blk
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.ent[mid].block_start <= blk) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The 16 bytes that start kb bytes (0..3) into dword j0 (0..3) of the
// 32-byte window lo:hi.
__device__ __forceinline__ u32x4 funnel(const u32x4 lo, const u32x4 hi, int j0, uint32_t kb) {
  const uint32_t d[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  u32x4 r;
  switch (j0) {
    case 0:
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(d[i + 1], d[i], kb);
      break;
    case 1:
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(d[i + 2], d[i + 1], kb);
      break;
    case 2:
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(d[i + 3], d[i + 2], kb);
      break;
    default:
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(d[i + 4], d[i + 3], kb);
      break;
  }
  return r;
}

template <int ESZ>
struct ElemT;
template <>
struct ElemT<2> { typedef gu16 T; };
template <>
struct ElemT<4> { typedef gu32 T; };

template <int ESZ>
__global__ void __launch_bounds__(kThreads) copy_kernel(const CopyArgs a) {
  typedef typename ElemT<ESZ>::T T;
  const int blk = blockIdx.x;
  const int ei = find_ent(a, blk);
  const uint64_t s_begin = (uint64_t)(uintptr_t)a.ent[ei].src;
  const bool zero_fill = s_begin == 0;
  const int64_t n = a.ent[ei].n;
  // The entry's destination bytes [d0, d1) and its 16-byte units.
  const uint64_t d0 = (uint64_t)(uintptr_t)a.dst + (uint64_t)a.ent[ei].dst_off * ESZ;
  const uint64_t d1 = d0 + (uint64_t)n * ESZ;
  const uint64_t u_end = (d1 + 15) >> 4;
  const uint64_t ublk =
      (d0 >> 4) + (uint64_t)(blk - a.ent[ei].block_start) * (kThreads * kCopyUnits);
  const uint64_t s_end = s_begin + (uint64_t)n * ESZ;
  const uint64_t shift = s_begin - d0;   // source byte = destination byte + shift (mod 2^64)

  // Interior workgroups -- every unit a whole 16-byte unit at least 16 bytes
  // inside the entry -- issue all their loads before any store, so each lane
  // keeps kCopyUnits loads in flight.  The source misalignment k is the same
  // for every unit of the entry, so the branches are uniform.
  constexpr uint64_t kStride = (uint64_t)kThreads * 16;   // bytes between a lane's units
  const uint64_t blk_lo = ublk << 4;
  const uint64_t blk_hi = blk_lo + kStride * kCopyUnits;
  if (blk_lo >= d0 + 16 && blk_hi + 16 <= d1) {
    const uint64_t ub0 = blk_lo + (uint64_t)threadIdx.x * 16;
    if (zero_fill) {
#pragma unroll
      for (int i = 0; i < kCopyUnits; ++i) st_nt(gaddr<gu32x4*>(ub0 + i * kStride), u32x4{0u, 0u, 0u, 0u});
      return;
    }
    const uint64_t p0 = ub0 + shift;
    const uint32_t k = (uint32_t)(p0 & 15);
    if (k == 0) {
      u32x4 r[kCopyUnits];
#pragma unroll
      for (int i = 0; i < kCopyUnits; ++i) r[i] = ld_nt(gaddr<const gu32x4*>(p0 + i * kStride));
#pragma unroll
      for (int i = 0; i < kCopyUnits; ++i) st_nt(gaddr<gu32x4*>(ub0 + i * kStride), r[i]);
    } else {
      // Both aligned loads of every unit lie inside the source: the unit is
      // at least 16 bytes from either end of the entry.
      const uint64_t a0 = p0 - k;
      u32x4 lo[kCopyUnits], hi[kCopyUnits];
#pragma unroll
      for (int i = 0; i < kCopyUnits; ++i) {
        lo[i] = ld_nt(gaddr<const gu32x4*>(a0 + i * kStride));
        hi[i] = ld_nt(gaddr<const gu32x4*>(a0 + i * kStride + 16));
      }
#pragma unroll
      for (int i = 0; i < kCopyUnits; ++i)
        st_nt(gaddr<gu32x4*>(ub0 + i * kStride), funnel(lo[i], hi[i], (int)(k >> 2), k & 3u));
    }
    return;
  }

  // Edge workgroups: unit by unit, partial units element by element.
#pragma unroll
  for (int i = 0; i < kCopyUnits; ++i) {
    const uint64_t u = ublk + (uint64_t)i * kThreads + threadIdx.x;
    if (u >= u_end) break;
    const uint64_t ub = u << 4;
    const uint64_t lo = ub > d0 ? ub : d0;
    const uint64_t hi = ub + 16 < d1 ? ub + 16 : d1;
    bool done = false;
    if (lo == ub && hi == ub + 16) {
      gu32x4* const up = gaddr<gu32x4*>(ub);
      if (zero_fill) {
        st_nt(up, u32x4{0u, 0u, 0u, 0u});
        done = true;
      } else {
        const uint64_t p = ub + shift;
        const uint32_t k = (uint32_t)(p & 15);
        if (k == 0) {
          st_nt(up, ld_nt(gaddr<const gu32x4*>(p)));
          done = true;
        } else {
          const uint64_t A = p - k;
          if (A >= s_begin && A + 32 <= s_end) {   // both aligned loads inside the source
            const u32x4 w0 = ld_nt(gaddr<const gu32x4*>(A));
            const u32x4 w1 = ld_nt(gaddr<const gu32x4*>(A + 16));
            st_nt(up, funnel(w0, w1, (int)(k >> 2), k & 3u));
            done = true;
          }
        }
      }
    }
    if (!done) {
      for (uint64_t b = lo; b < hi; b += ESZ) {
        *gaddr<T*>(b) = zero_fill ? 0 : *gaddr<const T*>(b + shift);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Warm-up read before the fused step
// ---------------------------------------------------------------------------

// Reads the given ranges of the step's fp32 state with ordinary (cached)
// loads and stores nothing; an empty asm takes each loaded value, so the
// loads are kept.  Run just before a large fused step it does two things on
// MI355X: the lines it brings into the 256 MB memory-side Infinity Cache push
// out what a producer of the gradients left there dirty (ordinary stores of
// the last ~256 MB written), so those write-backs happen now rather than
// among the step's reads; and the step then finds this part of its state in
// that cache.  After gradients written with ordinary stores the step is ~11%
// faster (7.5B, N_d = 64); after a step, or gradients written non-temporally,
// the step gains less than the read takes (1-2% net cost), which is why the
// read is opt-in.  Full workgroups take every unit without
// per-unit checks (wave w reads the workgroup's w-th 64 x kWarmUnits units
// as 1 KiB spans); the last workgroup of a range checks each unit.
__global__ void __launch_bounds__(kWarmThreads) warm_kernel(const WarmArgs a) {
  const int blk = blockIdx.x;
  int r = 0;
  for (int i = 1; i < a.n; ++i)
    if (a.block_start[i] <= blk) r = i;
  const int64_t units = a.units[r];
  const int64_t first = (int64_t)(blk - a.block_start[r]) * (kWarmThreads * kWarmUnits);
  const gu32x4* const p = gaddr<const gu32x4*>(a.base[r]);
  if (first + kWarmThreads * kWarmUnits <= units) {
    const gu32x4* const wv = p + first + (threadIdx.x >> 6) * (64 * kWarmUnits) + (threadIdx.x & 63);
    u32x4 x[kWarmUnits];
#pragma unroll
    for (int i = 0; i < kWarmUnits; ++i) x[i] = wv[i * 64];
#pragma unroll
    for (int i = 0; i < kWarmUnits; ++i) asm volatile("" ::"v"(x[i]));
  } else {
    for (int i = 0; i < kWarmUnits; ++i) {
      const int64_t u = first + threadIdx.x + (int64_t)i * kWarmThreads;
      if (u < units) {
        const u32x4 x = p[u];
        asm volatile("" ::"v"(x));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------

template <int MODE, int GDT, int PDT>
void* pick_ndc(int ndc) {
  switch (ndc) {
    case 4: return (void*)&step_vec_kernel<MODE, GDT, PDT, 4>;
    case 8: return (void*)&step_vec_kernel<MODE, GDT, PDT, 8>;
    case 16: return (void*)&step_vec_kernel<MODE, GDT, PDT, 16>;
    case 64: return (void*)&step_vec_kernel<MODE, GDT, PDT, 64>;
    default: return (void*)&step_vec_kernel<MODE, GDT, PDT, 0>;
  }
}

template <int MODE, int GDT, int PDT>
void* pick_step(int ndc, bool vec) {
  if (!vec) return (void*)&step_elem_kernel<MODE, GDT, PDT>;
  return pick_ndc<MODE, GDT, PDT>(ndc);
}

void* pick_kernel(int mode, int gdt, int pdt, int ndc, bool vec) {
  const bool gb = gdt == ZERO_BF16, pb = pdt == ZERO_BF16;
  if (mode == kFromReduced) {   // gradient type and rank count play no part
    if (pb) return vec ? (void*)&step_vec_kernel<kFromReduced, ZERO_BF16, ZERO_BF16, 1>
                       : (void*)&step_elem_kernel<kFromReduced, ZERO_BF16, ZERO_BF16>;
    return vec ? (void*)&step_vec_kernel<kFromReduced, ZERO_BF16, ZERO_F16, 1>
               : (void*)&step_elem_kernel<kFromReduced, ZERO_BF16, ZERO_F16>;
  }
  if (mode == kReduceOnly) {    // parameter type plays no part
    return gb ? pick_step<kReduceOnly, ZERO_BF16, ZERO_F16>(ndc, vec)
              : pick_step<kReduceOnly, ZERO_F16, ZERO_F16>(ndc, vec);
  }
  if (gb && pb) return pick_step<kFused, ZERO_BF16, ZERO_BF16>(ndc, vec);
  if (gb) return pick_step<kFused, ZERO_BF16, ZERO_F16>(ndc, vec);
  if (pb) return pick_step<kFused, ZERO_F16, ZERO_BF16>(ndc, vec);
  return pick_step<kFused, ZERO_F16, ZERO_F16>(ndc, vec);
}

}  // namespace

int launch_step(const StepArgs& a, int mode, int gdt, int pdt, int ndc, bool vec, int n_blocks,
                void* stream) {
  void* fn = pick_kernel(mode, gdt, pdt, ndc, vec);
  void* args[] = {(void*)&a};
  return (int)hipLaunchKernel(fn, dim3((unsigned)n_blocks), dim3(vec ? kStepThreads : kThreads), args,
                              0, (hipStream_t)stream);
}

int launch_copy(const CopyArgs& a, int esz, int n_blocks, void* stream) {
  void* fn = esz == 2 ? (void*)&copy_kernel<2> : (void*)&copy_kernel<4>;
  void* args[] = {(void*)&a};
  return (int)hipLaunchKernel(fn, dim3((unsigned)n_blocks), dim3(kThreads), args, 0,
                              (hipStream_t)stream);
}

int launch_warm(const WarmArgs& a, int n_blocks, void* stream) {
  void* args[] = {(void*)&a};
  return (int)hipLaunchKernel((void*)&warm_kernel, dim3((unsigned)n_blocks), dim3(kWarmThreads), args, 0,
                              (hipStream_t)stream);
}

int resident_blocks(int mode, int gdt, int pdt, int ndc, bool vec) {
  // Cached per kernel variant (all devices this library runs on are the same
  // gfx950 part); 0 = not yet known, -1 = query failed.
  static std::atomic<int> cache[3][3][3][5][2];
  const int ni = ndc == 4 ? 1 : ndc == 8 ? 2 : ndc == 16 ? 3 : ndc == 64 ? 4 : 0;
  std::atomic<int>& slot = cache[mode % 3][gdt % 3][pdt % 3][ni][vec ? 1 : 0];
  int r = slot.load(std::memory_order_relaxed);
  if (r != 0) return r < 0 ? 0 : r;
  int per_cu = 0, dev = 0, cus = 0;
  const void* fn = pick_kernel(mode, gdt, pdt, ndc, vec);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, vec ? kStepThreads : kThreads, 0) != hipSuccess ||
      hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    slot.store(-1, std::memory_order_relaxed);
    return 0;
  }
  r = per_cu * cus;
  slot.store(r > 0 ? r : -1, std::memory_order_relaxed);
  return r > 0 ? r : 0;
}

namespace {
// A positive integer attribute of the current device, cached per device and
// attribute slot; 0 if it cannot be read.
int device_attribute(int slot_id, hipDeviceAttribute_t attr) {
  constexpr int kDevices = 64, kSlots = 3;
  static std::atomic<int> cache[kDevices][kSlots];   // 0 = not yet known, -1 = query failed
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  std::atomic<int>* slot = dev >= 0 && dev < kDevices && slot_id < kSlots ? &cache[dev][slot_id] : nullptr;
  int v = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v <= 0) {
      (void)hipGetLastError();
      v = -1;
    }
    if (slot) slot->store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}
}  // namespace

double wall_clock_hz() { return 1e3 * device_attribute(0, hipDeviceAttributeWallClockRate); }

double hbm_peak_bps() {
  const double khz = device_attribute(1, hipDeviceAttributeMemoryClockRate);
  const double bits = device_attribute(2, hipDeviceAttributeMemoryBusWidth);
  return 1e3 * khz * 4.0 * bits / 8.0;
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace zk
