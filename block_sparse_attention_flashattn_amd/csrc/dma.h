// LDS DMA helpers shared by the attention kernels: buffer descriptors, 16-byte
// loads from a buffer straight into LDS (the `lds` bit of buffer_load), explicit
// vmcnt waits for them, and an LDS-only workgroup barrier.
#pragma once
#include "tile.h"

namespace bsa {

// Raw buffer descriptor over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ v4i make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4i{static_cast<int>(static_cast<uint32_t>(a)),
             static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffff), static_cast<int>(bytes),
             0x00020000};
}

// 16 bytes per lane from buffer offset `voff` into LDS at lds + 16 * lane.
// Issued as inline assembly so that the compiler's wait-count bookkeeping,
// which cannot tell LDS ring stages apart, does not drain the ring before
// every LDS read; the waits for these loads are the explicit vmcnt below.
// M0 (the LDS destination) is saved and restored inside the statement; an
// LDS-DMA load needs one wait state after the SALU write of M0 (the compiler
// does not insert it for inline assembly), hence the s_nop.
__device__ __forceinline__ void dma16(v4i desc, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(desc)
      : "memory");
}

// Four 16-byte-per-lane loads from buffer `desc` into the consecutive 1-KB LDS
// segments dst, dst + 1024, dst + 2048 and dst + 3072 under one M0: the
// immediate offset 1024 i moves the source and the LDS destination together,
// so load i takes the source offset v_i = (its source offset) - 1024 i, which
// the caller keeps non-negative.  The immediate is range-checked with the offset.
// NT: non-temporal loads, for data read once, so that the caches keep what is
// reused.
template <bool NT = false>
__device__ __forceinline__ void dma16x4(v4i desc, uint32_t v0, uint32_t v1, uint32_t v2,
                                        uint32_t v3, uint32_t dst) {
  uint32_t saved;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %6, 0 offen nt lds\n\t"
        "buffer_load_dwordx4 %3, %6, 0 offen offset:1024 nt lds\n\t"
        "buffer_load_dwordx4 %4, %6, 0 offen offset:2048 nt lds\n\t"
        "buffer_load_dwordx4 %5, %6, 0 offen offset:3072 nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(dst), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(desc)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
        "buffer_load_dwordx4 %3, %6, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %4, %6, 0 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %5, %6, 0 offen offset:3072 lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(dst), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(desc)
        : "memory");
  }
}

// s_waitcnt vmcnt(n): n vector-memory operations may still be outstanding.
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 16)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (n >= 8)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n >= 4)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 31] (larger n waits as for 31).
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n < 31 ? n : 31) {
#define BSA_VM_CASE(k) \
  case k:              \
    asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); \
    break;
    BSA_VM_CASE(0) BSA_VM_CASE(1) BSA_VM_CASE(2) BSA_VM_CASE(3) BSA_VM_CASE(4) BSA_VM_CASE(5)
    BSA_VM_CASE(6) BSA_VM_CASE(7) BSA_VM_CASE(8) BSA_VM_CASE(9) BSA_VM_CASE(10) BSA_VM_CASE(11)
    BSA_VM_CASE(12) BSA_VM_CASE(13) BSA_VM_CASE(14) BSA_VM_CASE(15) BSA_VM_CASE(16)
    BSA_VM_CASE(17) BSA_VM_CASE(18) BSA_VM_CASE(19) BSA_VM_CASE(20) BSA_VM_CASE(21)
    BSA_VM_CASE(22) BSA_VM_CASE(23) BSA_VM_CASE(24) BSA_VM_CASE(25) BSA_VM_CASE(26)
    BSA_VM_CASE(27) BSA_VM_CASE(28) BSA_VM_CASE(29) BSA_VM_CASE(30) BSA_VM_CASE(31)
#undef BSA_VM_CASE
  }
}


// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding global loads and stores, so tile loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Four 1-KB segments (rows 8s .. 8s+7, s = 0..3) of one 32-row half tile from
// buffer `desc` into LDS at dst: lane l's 16 bytes land at dst + 1024 s + 16 l.
// The immediate offset moves the source and the LDS destination together, so
// one M0 serves all four; `ve` addresses segments 0 and 2, `vo` segments 1 and
// 3 (their swizzle differs).  The immediate is range-checked with the offset.
__device__ __forceinline__ void dma_half(v4i desc, uint32_t ve, uint32_t vo, uint32_t dst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %4, 0 offen lds\n\t"
      "buffer_load_dwordx4 %3, %4, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %2, %4, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %3, %4, 0 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(dst), "v"(ve), "v"(vo), "s"(desc)
      : "memory");
}

// dma_half for the K half tile into kdst and the V half tile into kdst + HALFB
// (same source offsets, different buffers) under one M0 save/restore.
__device__ __forceinline__ void dma_kv_half(v4i kdesc, v4i vdesc, uint32_t ve, uint32_t vo,
                                            uint32_t kdst, uint32_t vdst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
      "buffer_load_dwordx4 %4, %5, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %3, %6, 0 offen lds\n\t"
      "buffer_load_dwordx4 %4, %6, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %6, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %6, 0 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(kdst), "s"(vdst), "v"(ve), "v"(vo), "s"(kdesc), "s"(vdesc)
      : "memory");
}

}  // namespace bsa
