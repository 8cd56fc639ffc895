// Device building blocks shared by the scan and compaction kernels (gfx950,
// wave64).  Nothing here is specific to one kernel:
//   - element formats: storage type, the type the combine runs in, exact
//     widening and round-to-nearest-even narrowing;
//   - the combine operators and their identities;
//   - a 64-lane inclusive scan built from DPP row shifts and row broadcasts;
//   - 16-byte vector loads/stores over an aligned "window" with element masks;
//   - tile descriptors for decoupled look-back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sca {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Combine operators.  `a` is always the EARLIER operand ("Tile operations and
// reductions", section "Why not just infer it from reduce?": a noncommutative
// combine receives the earlier subsequence on its left).  min/max are written
// as compare+select exactly as the running-max/min kernels of metaltile-std
// src/mlx/scan.rs do, so ties (e.g. +0 vs -0) yield the later operand; the
// compiler keeps them as v_cmp + v_cndmask (no v_min/v_max, whose signed-zero
// rules differ).  Integer add runs in the unsigned type: it wraps mod 2^w.
// Mul (the product scans of the same page, identity 1) is defined for the
// floating accumulation types only.
// ---------------------------------------------------------------------------
enum class Op : int { Add = 0, Min = 1, Max = 2, Mul = 3 };

template <class T> struct Limits;
template <> struct Limits<float> {
  static __device__ __forceinline__ float lowest() { return -__builtin_huge_valf(); }
  static __device__ __forceinline__ float highest() { return __builtin_huge_valf(); }
};
template <> struct Limits<double> {
  static __device__ __forceinline__ double lowest() { return -__builtin_huge_val(); }
  static __device__ __forceinline__ double highest() { return __builtin_huge_val(); }
};
template <> struct Limits<int32_t> {
  static __device__ __forceinline__ int32_t lowest() { return INT32_MIN; }
  static __device__ __forceinline__ int32_t highest() { return INT32_MAX; }
};
template <> struct Limits<uint32_t> {
  static __device__ __forceinline__ uint32_t lowest() { return 0u; }
  static __device__ __forceinline__ uint32_t highest() { return UINT32_MAX; }
};
template <> struct Limits<int64_t> {
  static __device__ __forceinline__ int64_t lowest() { return INT64_MIN; }
  static __device__ __forceinline__ int64_t highest() { return INT64_MAX; }
};
template <> struct Limits<uint64_t> {
  static __device__ __forceinline__ uint64_t lowest() { return 0ull; }
  static __device__ __forceinline__ uint64_t highest() { return UINT64_MAX; }
};

template <Op O, class W>
__device__ __forceinline__ W identity() {
  if constexpr (O == Op::Add) return W(0);
  else if constexpr (O == Op::Mul) return W(1);
  else if constexpr (O == Op::Min) return Limits<W>::highest();
  else return Limits<W>::lowest();
}

template <class W> struct Unsigned { using type = W; };
template <> struct Unsigned<int32_t> { using type = uint32_t; };
template <> struct Unsigned<int64_t> { using type = uint64_t; };

template <Op O, class W>
__device__ __forceinline__ W combine(W a, W b) {
  if constexpr (O == Op::Add) {
    if constexpr (std::is_same_v<W, float> || std::is_same_v<W, double>) {
      return a + b;
    } else {
      using U = typename Unsigned<W>::type;
      return (W)((U)a + (U)b);
    }
  } else if constexpr (O == Op::Mul) {
    static_assert(std::is_same_v<W, float> || std::is_same_v<W, double>, "product of floats only");
    return a * b;
  } else if constexpr (O == Op::Min) {
    return (a < b) ? a : b;
  } else {
    return (a > b) ? a : b;
  }
}

// ---------------------------------------------------------------------------
// Element formats: S is the storage type, W the type the combine runs in.
// 16-bit floats widen exactly to float32 and narrow with round-to-nearest-even
// (hardware v_cvt_pk_bf16_f32 / v_cvt_f16_f32 under the default rounding mode),
// per "Tile operations and reductions", section "Storage and arithmetic
// precision".
// ---------------------------------------------------------------------------
struct FmtF32 { using S = float;    using W = float; };
struct FmtF16 { using S = uint16_t; using W = float; };
struct FmtBF16 { using S = uint16_t; using W = float; };
struct FmtF64 { using S = double;   using W = double; };
struct FmtI32 { using S = int32_t;  using W = int32_t; };
struct FmtU32 { using S = uint32_t; using W = uint32_t; };
struct FmtI64 { using S = int64_t;  using W = int64_t; };
struct FmtU64 { using S = uint64_t; using W = uint64_t; };

template <class F>
__device__ __forceinline__ typename F::W widen(typename F::S s) {
  if constexpr (std::is_same_v<F, FmtBF16>) {
    return __builtin_bit_cast(float, (uint32_t)s << 16);
  } else if constexpr (std::is_same_v<F, FmtF16>) {
    return (float)__builtin_bit_cast(_Float16, s);
  } else {
    return s;
  }
}

template <class F>
__device__ __forceinline__ typename F::S narrow(typename F::W w) {
  if constexpr (std::is_same_v<F, FmtBF16>) {
    return __builtin_bit_cast(uint16_t, (__bf16)w);
  } else if constexpr (std::is_same_v<F, FmtF16>) {
    return __builtin_bit_cast(uint16_t, (_Float16)w);
  } else {
    return w;
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two adjacent outputs rounded and packed into one dword (lower address low).
template <class F>
__device__ __forceinline__ uint32_t narrow2(float a, float b) {
  f32x2 v = {a, b};
  if constexpr (std::is_same_v<F, FmtBF16>) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

// ---------------------------------------------------------------------------
// Lane exchange.  DPP moves operate on 32-bit registers; 64-bit values move as
// two halves.  Lanes whose DPP source is out of range (or whose row is masked
// off) receive `old`, which callers set to the identity: a shift with a
// defined boundary fill ("Tile operations and reductions", section "Logical
// exchange versus physical shuffle").
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK, class W>
__device__ __forceinline__ W dpp(W src, W old) {
  if constexpr (sizeof(W) == 4) {
    return __builtin_bit_cast(W, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, old), __builtin_bit_cast(int, src), CTRL, ROW_MASK, 0xf, false));
  } else {
    uint64_t s = __builtin_bit_cast(uint64_t, src), o = __builtin_bit_cast(uint64_t, old);
    uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)o, (int)(uint32_t)s,
                                                       CTRL, ROW_MASK, 0xf, false);
    uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(o >> 32),
                                                       (int)(uint32_t)(s >> 32), CTRL, ROW_MASK,
                                                       0xf, false);
    return __builtin_bit_cast(W, ((uint64_t)hi << 32) | lo);
  }
}

template <class W>
__device__ __forceinline__ W readlane(W v, int lane) {
  if constexpr (sizeof(W) == 4) {
    return __builtin_bit_cast(W, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
  } else {
    uint64_t u = __builtin_bit_cast(uint64_t, v);
    uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(W, ((uint64_t)hi << 32) | lo);
  }
}

// DPP control codes (GFX9 encoding).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

// Inclusive scan across the 64 lanes (lane i gets v_0 (+) ... (+) v_i).
// Steps 1-4 scan each 16-lane row (shift right by 1, 2, 4, 8 within the row);
// row_bcast:15 adds row 0's total into row 1 and row 2's into row 3;
// row_bcast:31 adds lane 31's prefix into rows 2 and 3.  The value that comes
// from a lower lane is always the left (earlier) operand.
template <Op O, class W>
__device__ __forceinline__ W wave_scan_incl(W v) {
  const W id = identity<O, W>();
  v = combine<O>(dpp<kRowShr1, 0xf>(v, id), v);
  v = combine<O>(dpp<kRowShr2, 0xf>(v, id), v);
  v = combine<O>(dpp<kRowShr4, 0xf>(v, id), v);
  v = combine<O>(dpp<kRowShr8, 0xf>(v, id), v);
  v = combine<O>(dpp<kRowBcast15, 0xa>(v, id), v);
  v = combine<O>(dpp<kRowBcast31, 0xc>(v, id), v);
  return v;
}

// Exclusive scan from an inclusive one: shift by one lane, lane 0 gets the
// identity.
template <Op O, class W>
__device__ __forceinline__ W wave_shift_excl(W incl) {
  return dpp<kWaveShr1, 0xf>(incl, identity<O, W>());
}

// Keeps v in registers as computed here: the compiler may not sink the
// arithmetic that produced it past this point (used to finish in-place
// updates before a barrier, so that their inputs die early).
template <class W>
__device__ __forceinline__ void materialize(W& v) {
  if constexpr (sizeof(W) == 8) {
    uint64_t u = __builtin_bit_cast(uint64_t, v);
    asm volatile("" : "+v"(u));
    v = __builtin_bit_cast(W, u);
  } else {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    asm volatile("" : "+v"(u));
    v = __builtin_bit_cast(W, u);
  }
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }
// Wave index within the workgroup, as a wave-uniform (scalar) value so that
// addresses and buffer resources derived from it stay in scalar registers.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// ---------------------------------------------------------------------------
// Window addressing.  Kernels address an array through a 16-byte-aligned base
// `abase` that lies `ph` elements before the array's first element; window
// element index i is array element i - ph.  Vector v of the window covers
// window elements [v*E, v*E + E) and is a naturally aligned 16-byte block
// (E = 16 / sizeof(S)); with E == 1 (arrays whose phases differ) a vector is
// one element.
//
// Loads go through a buffer resource whose range ends at the last vector that
// holds a valid element, so every load is issued unconditionally (no branch,
// hence no wait for one load before the next is issued) and a vector past the
// range reads as zero bits without touching memory.  The vectors at the two
// ends of a valid range may hold neighbouring elements: they are masked to
// the identity after the load (only the two end vectors of a range are
// partial, and a 16-byte block never straddles a page, so reading them is
// safe).  Full vectors are stored with one 16-byte nontemporal store; partial
// vectors element by element, touching only valid elements.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A global-memory (address space 1) pointer to T at integer address a.  Going
// through it, rather than a generic pointer, makes the compiler emit global_*
// instead of flat_* instructions, whose extra counter use would force waits.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gptr(uintptr_t a) {
  return (__attribute__((address_space(1))) T*)a;
}

struct Buf {
  __amdgpu_buffer_rsrc_t r;
  // [base, base + bytes): base must be wave-uniform; bytes is clamped to the
  // 32-bit range of a buffer resource (callers keep windows below 2 GiB).
  __device__ __forceinline__ Buf(uintptr_t base, int64_t bytes) {
    const int nrec = bytes <= 0 ? 0 : (bytes >= 0x7ffffff0 ? 0x7ffffff0 : (int)bytes);
    r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrec, 0x00020000);
  }
};

constexpr int kNT = 2;  // nontemporal cache policy for streaming loads
// Cache policy of full-vector buffer stores.
#ifndef SCA_STORE_AUX
#define SCA_STORE_AUX 2
#endif
constexpr int kStoreAux = SCA_STORE_AUX;

template <class S, int E>
struct VecIO {
  static_assert(E == 1 || E * sizeof(S) == 16, "a vector is one element or 16 bytes");
  // Raw storage bits of one vector.
  using Raw = std::conditional_t<E == 1, S, uint4>;

  // Vector at byte offset `off` of buffer b (zero bits when out of its range).
  static __device__ __forceinline__ Raw load(const Buf& b, uint32_t off) {
    if constexpr (E == 1) {
      if constexpr (sizeof(S) == 2) {
        return __builtin_bit_cast(S, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(b.r, off, 0, kNT));
      } else if constexpr (sizeof(S) == 4) {
        return __builtin_bit_cast(S, (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(b.r, off, 0, kNT));
      } else {
        return __builtin_bit_cast(S, __builtin_amdgcn_raw_buffer_load_b64(b.r, off, 0, kNT));
      }
    } else {
      return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(b.r, off, 0, kNT));
    }
  }

  template <class F>
  static __device__ __forceinline__ void unpack(const Raw r, typename F::W (&x)[E]) {
    if constexpr (E == 1) {
      x[0] = widen<F>(r);
    } else {
      const uint32_t d[4] = {r.x, r.y, r.z, r.w};
      if constexpr (sizeof(S) == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = widen<F>(__builtin_bit_cast(S, d[k]));
      } else if constexpr (sizeof(S) == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[2 * k] = widen<F>((S)(d[k] & 0xffffu));
          x[2 * k + 1] = widen<F>((S)(d[k] >> 16));
        }
      } else {
        x[0] = widen<F>(__builtin_bit_cast(S, ((uint64_t)d[1] << 32) | d[0]));
        x[1] = widen<F>(__builtin_bit_cast(S, ((uint64_t)d[3] << 32) | d[2]));
      }
    }
  }

  // unpack, with elements outside window range [lo, hi) replaced by `id`
  template <class F>
  static __device__ __forceinline__ void unpack_masked(const Raw r, int64_t e0, int64_t lo,
                                                       int64_t hi, typename F::W id,
                                                       typename F::W (&x)[E]) {
    unpack<F>(r, x);
#pragma unroll
    for (int k = 0; k < E; ++k) x[k] = (e0 + k >= lo && e0 + k < hi) ? x[k] : id;
  }

  template <class F>
  static __device__ __forceinline__ uint4 pack(const typename F::W (&y)[E]) {
    uint32_t d[4];
    if constexpr (sizeof(S) == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) d[k] = __builtin_bit_cast(uint32_t, narrow<F>(y[k]));
    } else if constexpr (sizeof(S) == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) d[k] = narrow2<F>(y[2 * k], y[2 * k + 1]);
    } else {
      const uint64_t a = __builtin_bit_cast(uint64_t, narrow<F>(y[0]));
      const uint64_t b = __builtin_bit_cast(uint64_t, narrow<F>(y[1]));
      d[0] = (uint32_t)a; d[1] = (uint32_t)(a >> 32);
      d[2] = (uint32_t)b; d[3] = (uint32_t)(b >> 32);
    }
    return uint4{d[0], d[1], d[2], d[3]};
  }

  // Narrow y and store it as the full vector at byte offset off of buffer b
  // (one nontemporal buffer store).  The offset always travels in the VGPR
  // operand with a zero soffset: with an SGPR soffset the compiler assumes
  // the store-data hazard cannot occur and lets the next instruction
  // overwrite the data registers at once, and on MI355X such stores were
  // measured to write some lanes' data from the following instruction.
  template <class F>
  static __device__ __forceinline__ void store_full(const Buf& b, uint32_t off,
                                                    const typename F::W (&y)[E]) {
    if constexpr (E == 1) {
      const S s = narrow<F>(y[0]);
      if constexpr (sizeof(S) == 2) {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, s), b.r, off, 0, kStoreAux);
      } else if constexpr (sizeof(S) == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, s), b.r, off, 0, kStoreAux);
      } else {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, s), b.r, off, 0, kStoreAux);
      }
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pack<F>(y)), b.r, off, 0,
                                             kStoreAux);
    }
  }

  // Narrow y and store the elements of vector v that lie in [lo, hi).
  template <class F>
  static __device__ __forceinline__ void store(uintptr_t abase, int64_t v, int64_t lo, int64_t hi,
                                               const typename F::W (&y)[E]) {
    const int64_t e0 = v * E;
    if constexpr (E == 1) {
      if (e0 >= lo && e0 < hi) *gptr<S>(abase + e0 * sizeof(S)) = narrow<F>(y[0]);
    } else {
      if (e0 >= lo && e0 + E <= hi) {
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, pack<F>(y)),
                                    gptr<u32x4>(abase + e0 * sizeof(S)));
      } else {
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const int64_t i = e0 + k;
          if (i >= lo && i < hi) *gptr<S>(abase + i * sizeof(S)) = narrow<F>(y[k]);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Tile descriptors for decoupled look-back.  Every descriptor word is one
// 64-bit value written once per call and read with the cache policy of
// relaxed agent-scope atomics (sc1), which on gfx950 is coherent across the
// XCDs' separate L2 caches.  Because a status and the value it qualifies
// always travel in the same word, no fence orders them.
//  - 32-bit values: one word  (status << 32) | value, one atomic store.
//  - 64-bit values: four words (aggregate lo/hi, inclusive lo/hi), each
//    (1 << 32) | half, a pair written by one 16-byte store; a reader accepts
//    a pair only when both halves are present, so it never mixes the two.
// Status: 0 = nothing yet, 1 = tile aggregate, 2 = inclusive prefix.
// A zero-filled descriptor array is the initial state.
// ---------------------------------------------------------------------------
enum : uint32_t { kNone = 0, kAgg = 1, kInc = 2 };

__device__ __forceinline__ void st_relaxed(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_relaxed(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Each tile's descriptor owns one 128-byte cache line (kDescLineWords words,
// of which kWords are used).  With descriptors packed 8 bytes apart, the
// tiles sharing a line contended for it while one wrote and many polled
// (MI355X, 2^28 i32 scan: 381 us packed, 367 us one line per tile; select
// of 2^28 f32 at p = 0.5: 406 us packed, 370 us per line).
constexpr int64_t kDescLineWords = 16;

template <class W, int SZ = sizeof(W)> struct Desc;

template <class W> struct Desc<W, 4> {
  static constexpr int kWords = 1;
  static __device__ __forceinline__ void publish(uint64_t* d, int64_t tile, uint32_t status, W v) {
    st_relaxed(d + tile * kDescLineWords,
               ((uint64_t)status << 32) | __builtin_bit_cast(uint32_t, v));
  }
  // Returns the status; sets v when it is not kNone.
  static __device__ __forceinline__ uint32_t read(const uint64_t* d, int64_t tile, W& v) {
    const uint64_t w = ld_relaxed(d + tile * kDescLineWords);
    v = __builtin_bit_cast(W, (uint32_t)w);
    return (uint32_t)(w >> 32);
  }
};

// 64-bit values: words 0-1 hold the aggregate, words 2-3 the inclusive
// prefix, each word (1 << 32) | half.  A pair is written with one 16-byte
// store and read with one 16-byte load, with the cache policy of the relaxed
// agent-scope atomics above (sc1), so both halves normally become visible
// together: written as two 8-byte stores, a poll that fell between them saw
// "not ready" and slept a whole pause, which cost 64-bit scans about 15 us
// of look-back at 2^26 elements.  Each 8-byte half is still single-copy
// atomic and carries its own flag, so a torn read is simply not ready.
template <class W> struct Desc<W, 8> {
  static constexpr int kWords = 4;
  static __device__ __forceinline__ void publish(uint64_t* d, int64_t tile, uint32_t status, W v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    uint64_t* slot = d + tile * kDescLineWords + (status == kInc ? 2 : 0);
    const u32x4 w = {(uint32_t)u, 1u, (uint32_t)(u >> 32), 1u};
    // The compiler's hazard checks do not see into asm: the wait states a
    // store of more than 8 bytes needs before its data registers may be
    // written again are part of the statement.
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 4" : : "v"(slot), "v"(w)
                 : "memory");
  }
  // Both pairs are loaded together (one round trip); the wait is part of the
  // load, so the poll is issued afresh every time.
  static __device__ __forceinline__ uint32_t read(const uint64_t* d, int64_t tile, W& v) {
    const uint64_t* s = d + tile * kDescLineWords;
    u32x4 a, i;
    asm volatile(
        "global_load_dwordx4 %0, %2, off sc1\n\t"
        "global_load_dwordx4 %1, %2, off offset:16 sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(a), "=&v"(i)
        : "v"(s)
        : "memory");
    if (i.y && i.w) {
      v = __builtin_bit_cast(W, ((uint64_t)i.z << 32) | i.x);
      return kInc;
    }
    if (a.y && a.w) {
      v = __builtin_bit_cast(W, ((uint64_t)a.z << 32) | a.x);
      return kAgg;
    }
    return kNone;
  }
};

// A data wave's part in publishing its tile's aggregate (called by lane 0 of
// each of the WD data waves, once): the wave posts its total to s_wave and
// counts itself in *s_posted; the last of the WD waves to do so combines the
// totals in wave order, publishes the tile's aggregate descriptor at once
// (tile 0 publishes its inclusive prefix instead, later) and raises
// *s_agg_done, after which the look-back wave may read s_wave and publish
// the inclusive prefix.  Publishing from the data side, rather than from the
// look-back wave between two of its polls, lets successors see the aggregate
// as soon as it exists; and because the inclusive prefix is only published
// after *s_agg_done, it can never be overwritten by the aggregate.
template <Op O, class W, int WD>
__device__ __forceinline__ void post_wave_total(W total, int wave, int64_t tile, W* s_wave,
                                                uint32_t* s_posted, uint32_t* s_agg_done,
                                                uint64_t* desc) {
  s_wave[wave] = total;
  const uint32_t before =
      __hip_atomic_fetch_add(s_posted, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (before == (uint32_t)WD - 1) {
    W a = s_wave[0];
#pragma unroll
    for (int w = 1; w < WD; ++w) a = combine<O>(a, s_wave[w]);
    if (tile > 0) Desc<W>::publish(desc, tile, kAgg, a);
    __hip_atomic_store(s_agg_done, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

__device__ __forceinline__ bool lds_flag_set(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_ACQUIRE,
                           __HIP_MEMORY_SCOPE_WORKGROUP) != 0u;
}

// Look-back by one wave: returns the combine of every tile before `tile`
// (the tile's exclusive prefix).  Lane l inspects tile base - 63 + l, so lane
// order is tile order and lane 63 is the nearest predecessor.  Each round
// waits until the lanes above the nearest inclusive descriptor (or all lanes,
// if there is none) hold at least an aggregate, reduces lanes
// [nearest inclusive .. 63] in order with the wave scan, and prepends the
// result to what later windows already gave.  Tiles before 0 read as
// inclusive identities, so the walk always ends.
//
// Waiting is bounded.  If a window's descriptors are not all published within
// `timeout` ticks of the 100 MHz real-time counter, the wave computes each
// missing tile's aggregate itself with reduce_tile(t) (a wave-cooperative
// reduction of tile t's input returning a wave-uniform value; the input never
// changes, so this is exactly what that tile would publish).  The walk then
// needs nothing from workgroups that have not started, so it ends whatever
// order the hardware runs workgroups in; in the usual case no descriptor is
// that late and no tile is reduced twice.
// Pause between two polls of a single descriptor (template argument PAUSE of
// look_back), in s_sleep units of 64 cycles.  The look-back only ever waits
// on one descriptor at a time (the nearest predecessor first, then the
// nearest one a window still lacks), so a poll is one load per wave, and
// windows of 64 descriptors are read only when the awaited one has arrived.
// Even so, frequent polls by hundreds of waiting tiles slow kernels whose
// tiles live long (2^28 i32 scan: 385 us at a pause of 8, 367 us at 127),
// while kernels with short-lived tiles need the finer wake-up (reduce-by-key
// of 2^27 pairs: 456 us at 8, 508 us at 127); each kernel passes its own.
constexpr int kPollLong = 127;   // about 8k cycles, ~3.4 us
constexpr int kPollShort = 8;    // about 512 cycles, ~0.2 us

template <Op O, class W, int PAUSE, class ReduceTile>
__device__ __forceinline__ W look_back(const uint64_t* desc, int64_t tile, uint64_t timeout,
                                       ReduceTile&& reduce_tile) {
  const int lane = lane_id();
  const W id = identity<O, W>();
  W prefix = id;
  {
    // Wait on the nearest predecessor alone first: it started last, so it is
    // usually the last to publish, and one descriptor per poll keeps the
    // polling traffic small while many tiles wait at once.
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    W v;
    while (Desc<W>::read(desc, tile - 1, v) == kNone &&
           __builtin_amdgcn_s_memrealtime() - t0 <= timeout)
      __builtin_amdgcn_s_sleep(PAUSE);
  }
  for (int64_t base = tile - 1;; base -= kWave) {
    const int64_t t = base - (kWave - 1) + lane;
    W v = id;
    uint32_t st = kNone;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
      st = (t < 0) ? (uint32_t)kInc : Desc<W>::read(desc, t, v);
      if (t < 0) v = id;
      const uint64_t inc = __ballot(st == kInc);
      const uint64_t none = __ballot(st == kNone);
      const uint64_t need = inc ? (~0ull << (63 - __builtin_clzll(inc))) : ~0ull;
      uint64_t pending = none & need;
      if (pending == 0) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > timeout) {
        while (pending) {                       // nearest missing tile first
          const int l = 63 - __builtin_clzll(pending);
          const W a = reduce_tile(base - (kWave - 1) + l);
          if (lane == l) {
            v = a;
            st = kAgg;
          }
          pending &= ~(1ull << l);
        }
        break;
      }
      // wait on the nearest missing descriptor alone (one load per poll),
      // then read the whole window again
      const int64_t tl = base - (kWave - 1) + (63 - __builtin_clzll(pending));
      W u;
      while (Desc<W>::read(desc, tl, u) == kNone &&
             __builtin_amdgcn_s_memrealtime() - t0 <= timeout)
        __builtin_amdgcn_s_sleep(PAUSE);
    }
    const uint64_t inc = __ballot(st == kInc);
    const int stop = inc ? 63 - __builtin_clzll(inc) : 0;
    if (lane < stop) v = id;
    const W window = readlane(wave_scan_incl<O>(v), kWave - 1);
    prefix = combine<O>(window, prefix);
    if (inc) return prefix;
  }
}

// The live element count of a call: n_cap, or, when the caller keeps the
// count in device memory (the entry points that take a device count, so one
// captured graph serves every count up to a capacity), that count clamped to
// [0, n_cap].  Read once per wave; the same value in every lane.
__device__ __forceinline__ int64_t live_count(int64_t n_cap, const int32_t* n_dev) {
  if (n_dev == nullptr) return n_cap;
  const int64_t v = *n_dev;
  return v < 0 ? 0 : (v > n_cap ? n_cap : v);
}

// Wait bound of the look-back before it reduces a late predecessor itself,
// in ticks of the 100 MHz real-time counter.  Far above the latency of a
// published descriptor (microseconds), so in practice it only matters if a
// predecessor's workgroup has not been scheduled.
#ifndef SCA_LOOKBACK_TIMEOUT_TICKS
#define SCA_LOOKBACK_TIMEOUT_TICKS 20000ull  // 200 us
#endif
constexpr uint64_t kLookBackTimeout = SCA_LOOKBACK_TIMEOUT_TICKS;

}  // namespace sca
