// MFMA operand helpers shared by the chunkwise kernels (gfx950).
#pragma once

#include "common.h"

namespace gdr {

__device__ __forceinline__ bf16x8 ld8(const bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// Block permutation of a q/k row with NB 16-byte blocks (NB = 16: 256-byte
// rows spanning all 64 banks; NB = 8: 128-byte rows, two rows per bank
// sweep).  A ds_read_b128 is serviced in four passes of 16 lanes; lane l
// joins pass (l >> 5, parity of (l >> 2) & 7) (measured on gfx950 with the
// bank-conflict counter), so one pass holds rows lr with
// parity(lr >> 2) = p of lane group 2h and the other rows of group 2h + 1,
// whose natural blocks differ in bit 0.  The permutation maps each of those
// two row sets onto the even blocks (with the row parity for NB = 8), so a
// pass reads 16 distinct blocks.  The transposing reads of k^T (64 lanes,
// one 8-byte half) meet each bank pair four times, their minimum.
template <int NB>
__device__ __forceinline__ int swz_qk(int r) {
  if constexpr (NB == 16) return 2 * (r & 7);
  else return 2 * ((r >> 1) & 3);
}

// Block permutation of a v row (NB = 8: 128-byte rows; NB = 4: 64-byte
// rows): the transposing reads of 8 rows x 2 blocks x 2 halves then hit 32
// distinct bank pairs.
template <int NB>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (NB == 8) return r & 6;
  else return 2 * ((r >> 2) & 1);
}

// Byte offset of slot i of a rotating LDS buffer, as a wave-uniform value
// the compiler cannot strength-reduce: an LDS address in a loop is then one
// add of a scalar to a per-lane offset (the induction form takes two).
__device__ __forceinline__ int slot_off(int i, int bytes) {
  return __builtin_amdgcn_readfirstlane(i * bytes);
}
template <typename T>
__device__ __forceinline__ T *at_off(T *p, int bytes) {
  return reinterpret_cast<T *>(reinterpret_cast<char *>(p) + bytes);
}
template <typename T>
__device__ __forceinline__ const T *at_off(const T *p, int bytes) {
  return reinterpret_cast<const T *>(reinterpret_cast<const char *>(p) + bytes);
}

// Makes this wave's earlier LDS writes visible to its later LDS reads of
// other lanes' data (LDS serves one wave's accesses in order; the fences
// keep the compiler from moving accesses across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Split two fp32 values into packed bf16 hi and lo pairs (x ~= hi + lo to
// ~16 bits, hi = RNE(x), lo = RNE(x - hi)).  One packed conversion makes
// both hi values and x - hi is exact in fp32 (hi is x rounded to 8 bits); a
// second packed conversion makes the lo pair.
//
// x - hi takes one of two forms:
//  - DOT: one instruction per value, the packed bf16 dot product
//    hi . m + x with m = (-1, 0) or (0, -1) (bf16 -1.0 is 0xBF80; the
//    products are exact).  It goes through the compiler builtin, whose form
//    ties the accumulator to the destination (a copy of x first when x
//    stays live).  It must stay visible to the compiler: a VALU write of a
//    register that an MFMA issued just before still reads as its
//    accumulator input needs wait states, which the compiler inserts for
//    its own instructions but not for inline assembly.
//  - otherwise: the hi values unpacked by a shift and a mask, then
//    subtracted (two instructions per value, freely scheduled).
template <bool DOT = true>
__device__ __forceinline__ void split2(float x0, float x1, unsigned &hi, unsigned &lo) {
  const bf16x2 h = __builtin_convertvector(f32x2{x0, x1}, bf16x2);
  hi = __builtin_bit_cast(unsigned, h);
  float r0, r1;
  if constexpr (DOT) {
    // the masks reach the instruction from SGPRs: the compiler would fold
    // (-1, 0) into the inline constant -1.0, which the hardware does not
    // read as that bf16 pair
    unsigned m0 = 0x0000BF80u, m1 = 0xBF800000u;
    asm("" : "+s"(m0), "+s"(m1));
    r0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m0), x0, false);
    r1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m1), x1, false);
  } else {
    r0 = x0 - __builtin_bit_cast(float, hi << 16);
    r1 = x1 - __builtin_bit_cast(float, hi & 0xffff0000u);
  }
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
}

// split4 of two tiles whose values stay live after the split (the state):
// the same steps as split2, with x - hi from the three-operand packed dot
// product, whose result register is not tied to its accumulator input (the
// two-operand form that the builtin selects needs a copy of each x first).
// Written as one block of inline assembly, which takes on the wait states
// the compiler keeps for its own instructions on this target:
//  - the block starts with 4 wait states: a VALU write of a register that an
//    MFMA issued just before still reads as its accumulator input needs 3
//    (the compiler's own code keeps 3 after a 16x16x32 bf16 MFMA);
//  - a dot product's result may be read by another VALU instruction only 3
//    wait states after it is written: the eight products come first, then
//    the four conversions (each reads its inputs at least 3 later);
//  - an MFMA may read a VALU result 2 wait states after it is written: the
//    block ends with them.
// The assembly scan of the kernels checks the first and the last rule on
// every path.
__device__ __forceinline__ void split8_keep(const f32x4 a, const f32x4 b, bf16x8 &hi, bf16x8 &lo) {
  unsigned h[4];
  h[0] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a[0], a[1]}, bf16x2));
  h[1] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a[2], a[3]}, bf16x2));
  h[2] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{b[0], b[1]}, bf16x2));
  h[3] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{b[2], b[3]}, bf16x2));
  unsigned m0 = 0x0000BF80u, m1 = 0xBF800000u;
  asm("" : "+s"(m0), "+s"(m1));
  float r[8];
  unsigned l[4];
  asm("s_nop 3\n\t"
      "v_dot2_f32_bf16 %4, %12, %16, %18\n\t"
      "v_dot2_f32_bf16 %5, %12, %17, %19\n\t"
      "v_dot2_f32_bf16 %6, %13, %16, %20\n\t"
      "v_dot2_f32_bf16 %7, %13, %17, %21\n\t"
      "v_dot2_f32_bf16 %8, %14, %16, %22\n\t"
      "v_dot2_f32_bf16 %9, %14, %17, %23\n\t"
      "v_dot2_f32_bf16 %10, %15, %16, %24\n\t"
      "v_dot2_f32_bf16 %11, %15, %17, %25\n\t"
      "v_cvt_pk_bf16_f32 %0, %4, %5\n\t"
      "v_cvt_pk_bf16_f32 %1, %6, %7\n\t"
      "v_cvt_pk_bf16_f32 %2, %8, %9\n\t"
      "v_cvt_pk_bf16_f32 %3, %10, %11\n\t"
      "s_nop 1"
      : "=&v"(l[0]), "=&v"(l[1]), "=&v"(l[2]), "=&v"(l[3]), "=&v"(r[0]), "=&v"(r[1]),
        "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "s"(m0), "s"(m1), "v"(a[0]), "v"(a[1]),
        "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]));
  typedef unsigned u32x4_ __attribute__((ext_vector_type(4)));
  hi = __builtin_bit_cast(bf16x8, u32x4_{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4_{l[0], l[1], l[2], l[3]});
}

template <bool DOT = true>
__device__ __forceinline__ void split4(const f32x4 x, bf16x4 &hi, bf16x4 &lo) {
  unsigned h01, l01, h23, l23;
  split2<DOT>(x[0], x[1], h01, l01);
  split2<DOT>(x[2], x[3], h23, l23);
  hi = __builtin_bit_cast(bf16x4, u32x2{h01, h23});
  lo = __builtin_bit_cast(bf16x4, u32x2{l01, l23});
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ds_read_b64_tr_b16: within each group of 16 lanes, output lane i receives
// element (i & 3) of the 8-byte chunks addressed by lanes (i >> 2) + 4c,
// c = 0..3.  Pointing lane j of a group at &X[t_(j >> 2)][c0 + 4 (j & 3)]
// therefore hands lane i the column c0 + i of rows t_0..t_3: a transposed
// 4x16 fragment, straight from a row-major tile.
__device__ __forceinline__ bf16x4 ld_tr4(const bf16 *p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s *)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Raw buffer access (gfx9 descriptor: 32-bit data format, no stride).  The
// descriptor covers [base, base + bytes): loads past the end return zero and
// stores past it are dropped, so a descriptor based at a chunk's first row
// bounds every access by the end of the tensor.  Offsets are in bytes; the
// scalar offset stays 0 so the bounds check sees the whole offset.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Descriptor of a range known to be shorter than 4 GiB (no clamp: a 64-bit
// clamp compiles to VALU compares that the scalar code then waits for).
__device__ __forceinline__ rsrc_t make_rsrc32(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// a bf16 value, left as its 16 bits (converted where it is used, so that a
// load issued ahead is not waited for at once)
__device__ __forceinline__ unsigned buf_ld_u16(rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, __builtin_bit_cast(int, off), 0, 0);
}
// four adjacent bf16 values (8 bytes) as two dwords
__device__ __forceinline__ u32x2 buf_ld_b64(rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                       r, __builtin_bit_cast(int, off), 0, 0));
}
__device__ __forceinline__ float bf16_bits_to_f32(unsigned u) {
  return __builtin_bit_cast(float, u << 16);
}
// (offsets are the unsigned 32-bit buffer offset, passed through bit for bit)
__device__ __forceinline__ void buf_st1(float x, rsrc_t r, unsigned off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r,
                                        __builtin_bit_cast(int, off), 0, 0);
}
__device__ __forceinline__ void buf_st1(bf16 x, rsrc_t r, unsigned off) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r,
                                        __builtin_bit_cast(int, off), 0, 0);
}

// four adjacent values of a row at a global address, fp32 or bf16 (rounded
// to nearest even): one 16-byte or 8-byte store
__device__ __forceinline__ void st4(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }
__device__ __forceinline__ void st4(bf16 *p, f32x4 x) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  *reinterpret_cast<bf16x4_t *>(p) = __builtin_convertvector(x, bf16x4_t);
}

// four adjacent output values of a row in one 16-byte (fp32) or 8-byte
// (bf16) store
__device__ __forceinline__ void buf_st4(f32x4 x, rsrc_t r, unsigned off, float) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r,
                                         __builtin_bit_cast(int, off), 0, 0);
}
__device__ __forceinline__ void buf_st4(f32x4 x, rsrc_t r, unsigned off, bf16) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  const bf16x4_t h = __builtin_convertvector(x, bf16x4_t);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, h), r,
                                        __builtin_bit_cast(int, off), 0, 0);
}

// D += A(16x16) * B(16x16), bf16 operands, fp32 accumulate: lane l holds
// A[l & 15][4 (l >> 4) .. +3] and B[4 (l >> 4) .. +3][l & 15]; the result
// lane l holds D[4 (l >> 4) + e][l & 15] -- the B operand layout, so an
// accumulator split into bf16 feeds the next product's B side directly.
__device__ __forceinline__ f32x4 mfma16_bf16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ---- LDS DMA: buffer loads that write LDS directly ----
//
// buffer_load_dword{,x4} ... lds writes lane l's 4 (16) bytes to LDS at
// M0 + 4 l (M0 + 16 l): a wave moves one contiguous 256 B (1 KiB) run of
// LDS, while each lane's global offset is free, so a layout in LDS is chosen
// through the per-lane offsets.  Offsets past the descriptor's size read as
// zero.  The loads are issued from inline assembly, so the compiler neither
// tracks them nor waits on them before later LDS reads of the issuing wave:
// the issuing wave waits with wait_vmcnt() before a barrier that publishes
// the data.  M0 is saved and restored around the load (the compiler owns
// it); an SALU write of M0 takes one wait state before the load reads it.

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// gfx9 raw buffer descriptor as four scalar dwords (stride 0, 32-bit data)
// of a range known to be shorter than 4 GiB
__device__ __forceinline__ u32x4 rsrc_words(const void *base, unsigned bytes) {
  const unsigned long long a = (unsigned long long)base;
  return u32x4{(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a),
               (unsigned)__builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xffffu)),
               (unsigned)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}

// byte address of an LDS object (wave-uniform)
__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return (unsigned)__builtin_amdgcn_readfirstlane(
      (int)(unsigned)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}

__device__ __forceinline__ void lds_dma16(u32x4 r, unsigned voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(r)
      : "memory");
}

__device__ __forceinline__ void lds_dma4(u32x4 r, unsigned voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(r)
      : "memory");
}

// s_waitcnt vmcnt(N) (other counters untouched)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// sum over the 16 lanes of each row of a wave (lanes 16 j .. 16 j + 15)
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}
__device__ __forceinline__ float sum64(float x) {
  x = sum16(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// The backward's workspace in fragment order.  A chunk's D x D state (h or
// dh; k channel c, value column v) and its C x D tiles (U or dY; row r,
// column v) are stored in the order the chunk kernels' state waves hold
// them, so that each of their store instructions writes 256 contiguous
// bytes (row-major, a wave's 16 columns would be four 64-byte pieces of
// different lines).  With c = 32 (mb >> 1) + 8 g + 4 (mb & 1) + e (the
// state waves' row order) and r = 16 rb + 4 g + e, the elements sit at
//   state (c, v): (((v >> 4) D/16 + mb) 4 + e) 4 + g) 16 + (v & 15)
//   tile  (r, v): (((v >> 4) C/16 + rb) 4 + e) 4 + g) 16 + (v & 15)
// Eight consecutive v of one c (or r) inside a 16-column block stay
// contiguous: the gradient kernels' operand reads.
__device__ __forceinline__ int ws_frag(int nblk, int vb, int mb, int e, int g, int l) {
  return (((vb * nblk + mb) * 4 + e) * 4 + g) * 16 + l;
}
__device__ __forceinline__ int ws_state_off(int D, int c, int v) {
  return ws_frag(D >> 4, v >> 4, 2 * (c >> 5) + ((c >> 2) & 1), c & 3, (c >> 3) & 3, v & 15);
}
__device__ __forceinline__ int ws_tile_off(int C, int r, int v) {
  return ws_frag(C >> 4, v >> 4, r >> 4, r & 3, (r >> 2) & 3, v & 15);
}

}  // namespace gdr
