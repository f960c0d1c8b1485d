// Asynchronous global -> LDS tile copies for gfx950 (global_load_lds_dwordx4).
//
// One instruction moves 16 bytes per lane straight into LDS at
// (wave-uniform base) + 16 * lane, without passing through VGPRs, and counts
// in the wave's vmcnt until the data has landed in LDS.  A tile of R rows of
// W 16-byte pieces is stored XOR-swizzled: piece c of row r lives at
// r * W + (c ^ (r & (min(W, 8) - 1))), so 16-byte fragment reads of 8
// consecutive rows at the same column hit distinct banks.
#pragma once
#include "device_common.hpp"

namespace msgla {

typedef __attribute__((address_space(3))) void lds_void_t;

// One 16-byte-per-lane asynchronous copy global -> LDS (a __device__ wrapper:
// kernels that name the builtin directly get no host-side launch stub).
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}

__device__ __forceinline__ int swz(int r, int c, int W) { return c ^ (r & ((W < 8 ? W : 8) - 1)); }

// byte offset of piece (r, c) in a swizzled tile of W pieces per row
__device__ __forceinline__ int swz_off(int r, int c, int W) { return (r * W + swz(r, c, W)) * 16; }

// Copies rows x W pieces (row stride gstride bytes) into the swizzled LDS tile.
// Waves [0, nwaves) split the 64-piece instructions round-robin; returns the
// number of instructions this wave issued (wave-uniform).
__device__ __forceinline__ int copy_tile_async(const char* g, size_t gstride, int rows, int W,
                                               char* lds, int wave, int nwaves, int lane) {
  const int n_instr = rows * W / 64;
  int issued = 0;
  for (int k = wave; k < n_instr; k += nwaves) {
    const int p = 64 * k + lane;
    const int r = p / W, pc = p - r * W;
    const int c = swz(r, pc, W);  // the XOR is an involution: phys pc <-> logical c
    __builtin_amdgcn_global_load_lds(g + (size_t)r * gstride + c * 16,
                                     (lds_void_t*)(lds + 64 * 16 * k), 16, 0, 0);
    ++issued;
  }
  return issued;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// runtime-count version (n is wave-uniform); counts above 63 wait for 63
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
#define MSGLA_W4(b) \
  case b: wait_vmcnt<b>(); break; case b + 1: wait_vmcnt<b + 1>(); break; \
  case b + 2: wait_vmcnt<b + 2>(); break; case b + 3: wait_vmcnt<b + 3>(); break;
  switch (n < 0 ? 0 : (n > 63 ? 63 : n)) {
    MSGLA_W4(0) MSGLA_W4(4) MSGLA_W4(8) MSGLA_W4(12) MSGLA_W4(16) MSGLA_W4(20) MSGLA_W4(24)
    MSGLA_W4(28) MSGLA_W4(32) MSGLA_W4(36) MSGLA_W4(40) MSGLA_W4(44) MSGLA_W4(48) MSGLA_W4(52)
    MSGLA_W4(56) MSGLA_W4(60)
    default: wait_vmcnt<0>(); break;
  }
#undef MSGLA_W4
}


// ---- contiguous tiles viewed as rows of 128 bytes ---------------------------
// A contiguous block holding logical rows of 2^lg bytes is stored in LDS as
// "virtual rows" of 128 bytes (8 pieces of 16 bytes), each piece index XORed
// with a key that changes from one logical row to the next (for rows of at
// least 128 bytes the key is the logical row & 7; shorter rows share a virtual
// row and use its index).  16-byte reads of one piece of 8 consecutive logical
// rows then hit distinct banks.  The copy is a plain contiguous DMA in which
// each lane picks the global piece that belongs in its LDS slot.
__device__ __forceinline__ int blk_hs(int lg) { return lg >= 7 ? lg - 7 : 0; }

// LDS byte offset of 16-byte piece p of logical row r (rows of 2^lg bytes)
__device__ __forceinline__ int tile_off(int r, int p, int lg) {
  int vrow, piece, hs;
  if (lg >= 7) {
    hs = lg - 7;
    vrow = (r << hs) + (p >> 3);
    piece = p & 7;
  } else {
    const int g = 7 - lg;
    hs = 0;
    vrow = r >> g;
    piece = ((r & ((1 << g) - 1)) << (lg - 4)) + p;
  }
  return vrow * 128 + ((piece ^ ((vrow >> hs) & 7)) << 4);
}

// Issue this wave's share (instructions k = wave, wave + nw, ...) of the copy of
// a contiguous block of `bytes` bytes; returns the number of instructions issued.
__device__ __forceinline__ int dma_block(const char* g, int bytes, int lg, char* lds, int wave,
                                        int nw, int lane) {
  const int hs = blk_hs(lg);
  const int n_instr = (bytes + 1023) >> 10;
  int issued = 0;
  for (int k = wave; k < n_instr; k += nw) {
    const int vrow = 8 * k + (lane >> 3);
    const int piece = (lane & 7) ^ ((vrow >> hs) & 7);  // global piece for this LDS slot
    if (vrow * 128 + 16 * (lane & 7) < bytes)
      __builtin_amdgcn_global_load_lds(g + vrow * 128 + piece * 16,
                                       (lds_void_t*)(lds + 1024 * k), 16, 0, 0);
    ++issued;
  }
  return issued;
}

// Workgroup barrier that waits for this wave's LDS operations only
// (lgkmcnt(0)); global loads and LDS-DMA copies still in flight are not
// waited for (__syncthreads() would wait for all of them, vmcnt(0)).  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace msgla
