// The bf16 / e4m3 GEMM kernel: the same contraction and fused epilogues as gemm_kernel.hpp,
// with operands moved HBM -> LDS by the LDS-DMA form of the global load (no VGPR staging, no
// LDS store instructions) through a ring of LDS stages, and a software-pipelined MFMA loop.
//
// Per workgroup (4 wave64 in 2 x 2, or 8 in 4 x 2 with two per SIMD; waves of WM x WN):
//  * one K-step is 128 bytes of K per operand row: 64 k for bf16 (four K=16 MFMA substeps),
//    128 k for e4m3 (two K=64 substeps); full 128-byte row segments keep every DMA request a
//    whole cache line;
//  * K-major operand tiles are [rows][ROWB], 16-byte chunks XOR-swizzled by row;
//  * MN-major operand tiles (bf16) are [64 k-rows][rows * 2 B], chunks XOR-swizzled by
//    (k-row % 4); fragments come out through the transposing 64-bit LDS read, which hands each
//    lane four consecutive k of one column;
//  * the ring holds NS K-steps. The DMA of step kt+NS is issued right after the barrier that
//    ends step kt's reads, into the stage step kt used, so NS-1 steps are in flight while one
//    is multiplied: the load latency of the shared L2 / last-level cache is hidden by depth.
//    Inside a step the fragments of substep s+1 are read while the MFMAs of substep s run;
//  * a DMA address is a wave-uniform base (SGPRs) plus a 32-bit per-lane offset; in the 8-wave
//    tiles with a K-major A, one wave per SIMD issues all of a step's DMAs.
#pragma once

#include <climits>
#include <type_traits>
#include <utility>

#include "epilogue_rows.hpp"
#include "gemm_kernel.hpp"

namespace gmlp {

// The DMA source of every tile slot that lies outside a matrix: 16 zero bytes.
static __device__ __attribute__((aligned(16))) uint32_t g_zero_chunk[4];

#define GMLP_LDS(p) ((__attribute__((address_space(3))) char*)(p))

// One LDS-DMA instruction: lane l's 16 bytes at src land at lds_wave_base + 16 l (the base is
// wave-uniform and goes in M0). Issued as inline assembly on purpose: for the compiler's own
// LDS-DMA builtin, the waitcnt pass cannot tell the DMA's LDS destination apart from a later
// transposing LDS read and waits for every DMA in flight before each such read, which would
// serialise the ring. The kernel counts its DMAs itself (wait_vmcnt), and the memory clobber
// keeps every LDS access in program order around the issue.
__device__ __forceinline__ void dma16(const void* src, char* lds_wave_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)GMLP_LDS(lds_wave_base);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}

// The same DMA with the address split into a wave-uniform 64-bit base (SGPRs) and a per-lane
// 32-bit byte offset (one VGPR instead of a 64-bit pointer per lane).
__device__ __forceinline__ void dma16s(const char* base, uint32_t voff, char* lds_wave_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)GMLP_LDS(lds_wave_base);
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// A uniform address the optimizer may not look through: the per-lane sum opaque(base + step) +
// offset then stays inside the K loop instead of being re-associated into a loop-invariant
// 64-bit base + offset per lane and hoisted (which would cost two VGPRs per DMA).
__device__ __forceinline__ const char* opaque_sgpr(const char* p) {
  asm("" : "+s"(p));
  return p;
}

// vmcnt(N), N < 64 (gfx9 encoding: low 4 bits in [3:0], high 2 bits in [15:14]); expcnt and
// lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Scheduling pattern for one substep region: each MFMA is followed by its share of the LDS
// reads of the next substep (and of the DMAs of a later K-step), so memory instructions issue
// between MFMAs instead of stalling the matrix pipe.
template <int I, int NM, int ND, int NV>
__device__ __forceinline__ void interleave_step() {
  constexpr int RP = (ND + NM - 1) / NM, VP = (NV + NM - 1) / NM;   // per MFMA slot
  constexpr int R = ND - I * RP < RP ? (ND - I * RP > 0 ? ND - I * RP : 0) : RP;
  constexpr int V = NV - I * VP < VP ? (NV - I * VP > 0 ? NV - I * VP : 0) : VP;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // MFMA
  if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // LDS reads
  if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x010, V, 0);  // VMEM (the DMAs)
}
template <int NM, int ND, int NV, int... I>
__device__ __forceinline__ void interleave_seq(std::integer_sequence<int, I...>) {
  (interleave_step<I, NM, ND, NV>(), ...);
}
template <int NM, int ND, int NV>
__device__ __forceinline__ void interleave() {
  interleave_seq<NM, ND, NV>(std::make_integer_sequence<int, NM>{});
}

// Scheduling pattern of a rolling substep: per column block j, its MI MFMAs, then the refill of
// B fragment j (RB LDS reads) and one of the NRA reads of the next substep's A fragments.
template <int J, int MI, int RB, int NRA>
__device__ __forceinline__ void interleave_roll_step() {
  __builtin_amdgcn_sched_group_barrier(0x008, MI, 0);                            // MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, RB + (J < NRA ? 1 : 0), 0);       // LDS reads
}
template <int MI, int RB, int NRA, int... J>
__device__ __forceinline__ void interleave_roll_seq(std::integer_sequence<int, J...>) {
  (interleave_roll_step<J, MI, RB, NRA>(), ...);
}
template <int MI, int NI, int RB, int NRA>
__device__ __forceinline__ void interleave_roll() {
  static_assert(NRA <= NI, "A reads spread one per column block");
  interleave_roll_seq<MI, RB, NRA>(std::make_integer_sequence<int, NI>{});
}

// Bytes of K per operand row in one K-step.
template <typename T> struct StepGeo;
template <> struct StepGeo<bf16> { static constexpr int ROWB = 128; };
template <> struct StepGeo<f16> { static constexpr int ROWB = 128; };
template <> struct StepGeo<e4m3> { static constexpr int ROWB = 128; };
template <> struct StepGeo<f8g> { static constexpr int ROWB = 128; };

// ---- K-major operand: ROWS rows x ROWB bytes per stage -------------------------------------
// One DMA instruction fills 1 KB = 8 rows of 128 bytes: lane l -> row 8 j + l / 8, slot l % 8,
// which holds the row's logical chunk slot ^ swz(row). A tile row comes from one of two bases
// (the gate / up halves of a gated tile, or two matrices stacked along the rows): rows below
// split_row from base0, the rest from base1, each base shifted so tile row r sits r row pitches
// past it. With every row of the tile inside its matrix (interior), the lane part of an address
// depends on the instruction only through the parity of j (the swizzle's row bit 3), so a lane
// keeps two 32-bit offsets and the rest of each address is wave-uniform scalar arithmetic.
template <typename T, int ROWS, int WAVES>
struct KTileDma {
  static constexpr int ES = ElemTraits<T>::bytes;
  static constexpr int E = 16 / ES;
  static constexpr int ROWB = StepGeo<T>::ROWB;
  static constexpr int CPR = ROWB / 16;
  static constexpr int RPI = 1024 / ROWB;            // rows per DMA instruction
  static constexpr int kInst = ROWS / RPI / WAVES;   // per wave per stage
  static_assert(ROWB == 128 && RPI == 8, "128-byte K-steps: 8 rows per DMA instruction");
  static_assert(kInst >= 1 && ROWS % (RPI * WAVES) == 0, "tile rows must split over the waves");
  uint32_t voff[2];           // per lane, interior tiles: offset within an even / odd instruction's rows
  const char* base0;          // uniform: the two bases at the split's first k
  const char* base1;
  int64_t ld_bytes;           // uniform row pitch (shared by both bases)
  int split_row;              // uniform: first tile row read from base1
  bool interior;              // uniform: no tile row is clamped

  // chunk swizzle: a row pair (2i, 2i + 1) shares the XOR (row >> 1) & 7. Measured with the
  // bank-conflict counter and read throughput on gfx950, this is conflict-free for every K-major
  // fragment read the kernels make (16x16x32: 16 rows x 4 chunks; 32x32x16 and 32x32x64: 32 rows
  // x 2 or 4 chunks), where XOR-ing with (row & 7) ^ ((row >> 3) & 1) put half of the 16x16x32
  // reads' cycles into bank conflicts (half the read bandwidth).
  static __device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
  static __device__ __forceinline__ int off(int row, int chunk) {
    return row * ROWB + ((chunk ^ swz(row)) << 4);
  }

  // b0, b1: the shifted bases at k = 0; split: first tile row from b1; locate(r) -> {which,
  // rel}: tile row r is `rel` row pitches past base `which` (rel = r unless the row is past its
  // matrix: such rows are given an existing row, as their products only reach output rows that
  // are never stored, so no row needs a zero fill). interior: locate(r) == {r >= split, r} for
  // every tile row. split must be a multiple of 8 (an instruction's rows share one base). An
  // instruction's rows 8 j + q (q = lane / 8) have swizzle (q >> 1) | ((j & 1) << 2).
  __device__ __forceinline__ void init(int lane, int kbeg, const char* b0, const char* b1, int64_t ld, int split,
                                       bool inner) {
    base0 = b0 + (int64_t)kbeg * ES;
    base1 = b1 + (int64_t)kbeg * ES;
    ld_bytes = ld;
    split_row = split;
    interior = inner;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      voff[par] = (uint32_t)((lane / CPR) * ld) + (uint32_t)((((lane % CPR) ^ ((lane / CPR) >> 1) ^ (par << 2))) * 16);
  }
  // scalar base of instruction i (rows 8 j ..) at K offset k_rel
  __device__ __forceinline__ const char* sbase(int wave, int i, int k_rel) const {
    const int r = RPI * (wave * kInst + i);
    return (r >= split_row ? base1 : base0) + (int64_t)r * ld_bytes + (int64_t)k_rel * ES;
  }
  // K-step at k_rel (relative to the split's first k) of a K range k_left long. An interior tile's
  // step wholly inside the range (all but the last partial step and the trailing zero steps; a
  // uniform test) is one scalar add per DMA; otherwise each lane places its row and chunk and
  // chunks past the range read the zero chunk.
  template <typename Locate>
  __device__ __forceinline__ void issue(char* tile, int wave, int lane, int k_rel, int k_left, Locate locate) const {
    if (interior && k_rel + ROWB / ES <= k_left) {
#pragma unroll
      for (int i = 0; i < kInst; ++i)
        dma16s(sbase(wave, i, k_rel), ((wave * kInst + i) & 1) ? voff[1] : voff[0], tile + (wave * kInst + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < kInst; ++i) issue_i(tile, wave, lane, i, k_rel, k_left, locate);
    }
  }
  // DMA i of an interior tile's K-step wholly in range (no per-lane work)
  __device__ __forceinline__ void issue_fast_i(char* tile, int wave, int i, int k_rel) const {
    dma16s(sbase(wave, i, k_rel), ((wave * kInst + i) & 1) ? voff[1] : voff[0], tile + (wave * kInst + i) * 1024);
  }
  // DMA i of issue(), placed and range-checked per lane (no branch)
  template <typename Locate>
  __device__ __forceinline__ void issue_i(char* tile, int wave, int lane, int i, int k_rel, int k_left,
                                          Locate locate) const {
    const int row = RPI * (wave * kInst + i) + lane / CPR;
    const int c = (lane % CPR) ^ swz(row);
    const int2 loc = locate(row);
    const char* b0k = opaque_sgpr(base0 + (int64_t)k_rel * ES);
    const char* b1k = opaque_sgpr(base1 + (int64_t)k_rel * ES);
    const char* src = (loc.x ? b1k : b0k) + ((int64_t)loc.y * ld_bytes + c * 16);
    dma16(k_rel + c * E < k_left ? (const void*)src : (const void*)g_zero_chunk, tile + (wave * kInst + i) * 1024);
  }
  static __device__ __forceinline__ u32x4 read(const char* tile, int row, int ch) {
    return *reinterpret_cast<const u32x4*>(tile + off(row, ch));
  }
  // The same read for row = rowbase + r with rowbase a multiple of 16: the swizzle of such a row
  // is that of r, so the address splits into a wave-uniform block base plus a lane offset that is
  // the same for every block (the block's position folds into the instruction's offset).
  static __device__ __forceinline__ u32x4 read_block(const char* tile, int rowbase, int r, int ch) {
    return *reinterpret_cast<const u32x4*>(tile + rowbase * ROWB + off(r, ch));
  }
};

// ---- MN-major bf16 operand: 64 k-rows x ROWS columns per stage --------------------------------
// The operand may be two matrices stacked along K (rows k < k_split from the first, the rest
// from the second, both with the same leading dimension). DMA instruction j fills KPI k-rows
// (lane l: k-row KPI j + q, q = 16 l / ROWB, 16-byte chunk slot c = (16 l % ROWB) / 16). The
// chunk's column depends on the instruction only through k-row bits 0, 1 and 3 (the swizzle), so
// a lane keeps one 32-bit offset per pattern of those bits (4 for 256-column tiles, 2 for 128) and
// the k-row base KPI j * pitch, the K-step and the jump to the second matrix are wave-uniform
// scalar arithmetic. With PAT false (DMAs issued one at a time between MFMAs, where each one's
// VALU work lands in the MFMA stream) a lane keeps one offset per instruction instead.
template <int ROWS, int WAVES, bool PAT = true>
struct MNTileDma {
  static constexpr int KROWS = 64;
  static constexpr int ROWB = ROWS * 2;               // bytes per k-row
  static constexpr int KPI = 1024 / ROWB;             // k-rows per DMA instruction
  static constexpr int kInst = KROWS * ROWB / 1024 / WAVES;   // per wave per stage
  static_assert(kInst >= 1, "tile too narrow");
  static_assert(KPI == 2 || KPI == 4 || KPI == 8, "64- to 256-column tiles");
  // instruction j's swizzle-relevant k-row bits (KPI j) & 0b1011 -> pattern index
  static constexpr int NPAT = KPI == 2 ? 4 : 2;
  static __device__ __forceinline__ int pattern(int j) {
    const int b = (KPI * j) & 0b1011;
    return KPI == 2 ? ((b >> 1) & 1) | (((b >> 3) & 1) << 1) : (b >> 3) & 1;
  }
  static __device__ __forceinline__ int pattern_row(int pat) {   // k-row KPI j of a j with this pattern
    return KPI == 2 ? 2 * (pat & 1) + 8 * (pat >> 1) : 8 * pat;
  }
  static constexpr int NOFF = PAT ? NPAT : kInst;
  uint32_t voff[NOFF];    // per lane: q * pitch + column bytes per pattern, or the whole offset per instruction
  const char* base;       // uniform: the first matrix at the split's first k, tile column 0
  int64_t ld_bytes;       // uniform pitch

  // k-rows kr .. kr+3 land in distinct 64-byte groups, and k-rows 8 apart (read in the same pass
  // by the 16x16 fragments) in distinct 32-byte halves of them
  static __device__ __forceinline__ int phys_chunk(int c, int kr) { return c ^ ((kr & 3) << 2) ^ (((kr >> 3) & 1) << 1); }

  // b: element (0, tile column 0) of the first matrix; ld: its row pitch in bytes; ncols: columns
  // of the matrix from tile column 0 on (a multiple of 8). Chunks of tile columns past the matrix
  // read its last chunk instead: their products only reach output columns that are never stored.
  __device__ __forceinline__ void init(int wave, int lane, const char* b, int64_t ld, int kbeg, int ncols) {
    base = b + (int64_t)kbeg * ld;
    ld_bytes = ld;
    const int q = lane * 16 / ROWB, c = (lane * 16 % ROWB) >> 4;
#pragma unroll
    for (int o = 0; o < NOFF; ++o) {
      const int kr = PAT ? pattern_row(o) + q : KPI * (wave * kInst + o) + q;
      const int col = min(phys_chunk(c, kr) * 8, ncols - 8);   // the XOR is an involution
      voff[o] = (uint32_t)((PAT ? q : kr) * ld) + (uint32_t)(col * 2);
    }
  }
  // offset of instruction i (j = wave kInst + i) from the K-step's base; kbase: the scalar part
  __device__ __forceinline__ int64_t kbase(int j) const { return PAT ? (int64_t)(KPI * j) * ld_bytes : 0; }
  __device__ __forceinline__ uint32_t voff_of(int i, int j) const {
    if constexpr (!PAT) return voff[i];
    const int pat = pattern(j);
    if constexpr (NPAT == 4) return pat & 2 ? (pat & 1 ? voff[3] : voff[2]) : (pat & 1 ? voff[1] : voff[0]);
    else return pat ? voff[1] : voff[0];
  }
  // K-step starting at k0 (absolute); step_off: byte offset of this K-step from the first;
  // second: distance from a k-row's address in the first matrix to its address in the second.
  // A step wholly inside [.., kend) and on one side of k_split (a uniform test) costs scalar
  // address arithmetic only; otherwise each k-row is placed and range-checked on its own.
  __device__ __forceinline__ void issue(char* tile, int wave, int lane, int k0, int kend, int64_t step_off, int k_split,
                                        int64_t second) const {
    if (k0 + KROWS <= kend && (k0 + KROWS <= k_split || k0 >= k_split)) {
      const char* b = base + step_off + (k0 >= k_split ? second : 0);
#pragma unroll
      for (int i = 0; i < kInst; ++i) {
        const int j = wave * kInst + i;
        dma16s(b + kbase(j), voff_of(i, j), tile + j * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kInst; ++i) issue_i(tile, wave, lane, i, k0, kend, step_off, k_split, second);
    }
  }
  // DMA i of a K-step wholly in range; b: the step's uniform base (base + step offset, plus the
  // jump to the second matrix when the step lies there)
  __device__ __forceinline__ void issue_fast_i(char* tile, int wave, int i, const char* b) const {
    const int j = wave * kInst + i;
    dma16s(b + kbase(j), voff_of(i, j), tile + j * 1024);
  }
  // DMA i of issue() alone, placed and range-checked per lane (no branch)
  __device__ __forceinline__ void issue_i(char* tile, int wave, int lane, int i, int k0, int kend, int64_t step_off,
                                          int k_split, int64_t second) const {
    const int j = wave * kInst + i;
    const int k = k0 + KPI * j + lane * 16 / ROWB;
    const char* s = opaque_sgpr(base + step_off + kbase(j)) + (k >= k_split ? second : 0) + voff_of(i, j);
    dma16(k < kend ? (const void*)s : (const void*)g_zero_chunk, tile + j * 1024);
  }
  // Fragment of the 32-column block starting at tile column cb, K substep s (16 k): lane l gets
  // the 8 consecutive k 8*(l/32) .. +7 of column cb + l%32, via two transposing reads of four
  // k each. In each 16-lane group, lane i points at k-row (i/4) of its four and columns
  // 4*(i%4) .. +3 of the group's 16.
  static __device__ __forceinline__ u32x4 read(const char* tile, int cb, int s, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int kr = 16 * s + 8 * (g >> 1) + (i >> 2);
    const int c = cb + 16 * (g & 1) + 4 * (i & 3);
    const int off0 = kr * ROWB + (phys_chunk(c >> 3, kr) << 4) + (c & 7) * 2;
    const int off1 = off0 + 4 * ROWB;                  // k-row + 4: same (k-row % 4)
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + off0)));
    const u32x2 v1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + off1)));
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3);
  }
  // Fragment of the 16-column block at tile column cb for the 16x16x32 MFMA, substep s (32 k):
  // lane l gets k 8*(l/16) .. +7 of column cb + l%16. Each 16-lane group covers its 8 k with two
  // transposing reads of four k-rows.
  static __device__ __forceinline__ u32x4 read16(const char* tile, int cb, int s, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int kr = 32 * s + 8 * g + (i >> 2);
    const int c = cb + 4 * (i & 3);
    const int off0 = kr * ROWB + (phys_chunk(c >> 3, kr) << 4) + (c & 7) * 2;
    const int off1 = off0 + 4 * ROWB;                  // k-row + 4: same (k-row % 4) and (k-row / 8)
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + off0)));
    const u32x2 v1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + off1)));
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3);
  }
};

// ---- MN-major 8-bit operand: 128 k-rows x ROWS columns per stage -------------------------------
// The fp8 weight-gradient products read their row-major operands ([tokens][columns] codes) along
// the tokens, i.e. MN-major. DMA instruction j fills KPI = 1024 / ROWS k-rows (lane l: k-row
// KPI j + l / CPR, CPR = ROWS / 16 chunks of 16 columns per k-row, physical chunk l % CPR holding
// logical chunk (l % CPR) ^ (k-row & 7)). Fragments come out through the 8-bit transposing LDS
// read, which hands each lane of a 16-lane group eight consecutive k of one column; the XOR puts
// the eight k-rows one such read gathers from a logical chunk into eight different chunk
// positions, which cover every LDS bank. In a 128-column tile an instruction's k-rows start at a
// multiple of 8, so a lane's swizzle, and its 32-bit offset, is the same for every instruction;
// in a 256-column tile (four k-rows per instruction) it alternates with the instruction's parity.
// Tile columns past the matrix read its last chunk (their products reach only outputs that are
// never stored), so the matrix width must be a multiple of 16 columns.
template <int ROWS, int WAVES>
struct MNTileDma8 {
  static constexpr int KROWS = 128;
  static constexpr int ROWB = ROWS;                      // bytes per k-row
  static constexpr int CPR = ROWB / 16;                  // 16-byte chunks per k-row
  static constexpr int KPI = 1024 / ROWB;                // k-rows per DMA instruction
  static constexpr int kInst = KROWS * ROWB / 1024 / WAVES;   // per wave per stage
  static_assert(ROWS == 128 || ROWS == 256, "128- or 256-column tiles");
  static_assert(kInst >= 1, "tile too narrow");
  static constexpr int NOFF = KPI == 8 ? 1 : 2;
  uint32_t voff[NOFF];    // per lane: k-row pitch + column bytes, per instruction parity
  const char* base;       // uniform: the matrix at the split's first k, tile column 0
  int64_t ld_bytes;       // uniform pitch

  static __device__ __forceinline__ int phys_chunk(int c, int kr) { return c ^ (kr & 7); }

  // b: element (0, tile column 0); ld: row pitch in bytes; ncols: columns of the matrix from tile
  // column 0 on (a multiple of 16)
  __device__ __forceinline__ void init(int, int lane, const char* b, int64_t ld, int kbeg, int ncols) {
    base = b + (int64_t)kbeg * ld;
    ld_bytes = ld;
    const int q = lane / CPR, p = lane % CPR;
#pragma unroll
    for (int o = 0; o < NOFF; ++o) {
      const int col = min(phys_chunk(p, KPI * o + q) * 16, ncols - 16);   // the XOR is an involution
      voff[o] = (uint32_t)(q * ld) + (uint32_t)col;
    }
  }
  __device__ __forceinline__ int64_t kbase(int j) const { return (int64_t)(KPI * j) * ld_bytes; }
  __device__ __forceinline__ uint32_t voff_of(int, int j) const {
    if constexpr (NOFF == 1) return voff[0];
    else return (j & 1) ? voff[1] : voff[0];
  }
  // K-step starting at k0 (absolute) of a range ending at kend; step_off: byte offset of this
  // K-step from the first. (No operand here is stacked along K: the last two arguments of the
  // 16-bit loader's interface are unused.)
  __device__ __forceinline__ void issue(char* tile, int wave, int lane, int k0, int kend, int64_t step_off, int,
                                        int64_t) const {
    if (k0 + KROWS <= kend) {
      const char* b = base + step_off;
#pragma unroll
      for (int i = 0; i < kInst; ++i) {
        const int j = wave * kInst + i;
        dma16s(b + kbase(j), voff_of(i, j), tile + j * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kInst; ++i) issue_i(tile, wave, lane, i, k0, kend, step_off, 0, 0);
    }
  }
  __device__ __forceinline__ void issue_fast_i(char* tile, int wave, int i, const char* b) const {
    const int j = wave * kInst + i;
    dma16s(b + kbase(j), voff_of(i, j), tile + j * 1024);
  }
  // DMA i of issue() alone, each k-row range-checked per lane (rows past kend load zeros)
  __device__ __forceinline__ void issue_i(char* tile, int wave, int lane, int i, int k0, int kend, int64_t step_off,
                                          int, int64_t) const {
    const int j = wave * kInst + i;
    const int k = k0 + KPI * j + lane / CPR;
    const char* src = opaque_sgpr(base + step_off + kbase(j)) + voff_of(i, j);
    dma16(k < kend ? (const void*)src : (const void*)g_zero_chunk, tile + j * 1024);
  }
  // The two 16-byte chunks of the 32-column block at tile column cb for the 32x32x64 MFMA,
  // substep s (64 k): lane l gets k 64 s + 32 (l / 32) .. +31 of column cb + l % 32, in k order,
  // from four transposing reads of eight k-rows. In each 16-lane group lane i points at k-row i / 2
  // of the read's eight and at bytes 8 (i % 2) .. +7 of the group's 16 columns; the read returns
  // to lane i column i of those eight k-rows.
  static __device__ __forceinline__ void read8(const char* tile, int cb, int s, int lane, u32x4& lo, u32x4& hi) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const int i = lane & 15, g = lane >> 4;
    const int c16 = (cb >> 4) + (g & 1);   // the group's logical chunk
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kr = 64 * s + 32 * (g >> 1) + 8 * j + (i >> 1);
      const int off = kr * ROWB + (phys_chunk(c16, kr) << 4) + 8 * (i & 1);
      const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(tile + off));
      w[2 * j] = (uint32_t)v[0];
      w[2 * j + 1] = (uint32_t)v[1];
    }
    lo = u32x4{w[0], w[1], w[2], w[3]};
    hi = u32x4{w[4], w[5], w[6], w[7]};
  }
};

// Stages in the ring: as many as fit the 160 KiB of LDS, at most 4; tiles of 128 x 128 and
// below keep room for two workgroups per CU (a second workgroup hides latency better than a
// deeper ring).
constexpr int ring_stages(int stage_bytes, int tile_elems) {
  const int lds = 160 * 1024;
  int n = lds / stage_bytes;
  if (tile_elems <= 128 * 128 && (lds / 2) / stage_bytes >= 2) n = (lds / 2) / stage_bytes;
  return n > 4 ? 4 : n;
}

// A stages beyond the ring's NS: tiles of 128 x 128 and below (two workgroups per CU) run few
// MFMAs per K-step, so in their large-M products (the fp8 GEMMs of the GPT-shape MLP, where A is
// streamed from HBM and B, the weights, stays in L2) each step waited on its A operand; the
// 16 KB their two-stage ring leaves of half the LDS hold one more A stage.
template <typename T, int BM, int BN>
constexpr int extra_a_stages() {
  constexpr int stage = (BM + BN) * StepGeo<T>::ROWB, a = BM * StepGeo<T>::ROWB;
  constexpr int ns = ring_stages(stage, BM * BN);
  return (BM * BN <= 128 * 128 && ns < 4 && ns * stage + a <= 80 * 1024) ? 1 : 0;
}

// LDS of one workgroup's ring (NS stages of a BM x BN tile's K-step, plus the extra A stages).
template <typename T, int BM, int BN>
constexpr int dma_ring_bytes() {
  constexpr int stage = (BM + BN) * StepGeo<T>::ROWB;
  return ring_stages(stage, BM * BN) * stage + extra_a_stages<T, BM, BN>() * BM * StepGeo<T>::ROWB;
}

// One output tile of a GEMM: tile `item` of p's grid (tiles_m x tiles_n x splits, the split
// index major), with `smem` the workgroup's LDS ring of dma_ring_bytes<T, BM, BN>() bytes.
// WAVES = 4: 2 x 2 waves, one per SIMD (wave tile up to 128 x 128, 256 accumulator registers).
// WAVES = 8: 4 x 2 waves, two per SIMD, so one wave's MFMAs fill the other's stalls (wave tile
// 64 x 128, 128 accumulator registers, half the register file each).
template <typename T, typename IoT, int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI, int WAVES>
__device__ __forceinline__ void gemm_dma_tile(const GemmArgs p, int item, char* smem) {
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must split into 2x2 waves of 32x32 blocks");
  static_assert((A_KMAJ && B_KMAJ) || ElemTraits<T>::bytes == 2 || (WAVES == 4 && !A_KMAJ && !B_KMAJ),
                "8-bit operands are MN-major only in 4-wave TN tiles");
  constexpr int ES = ElemTraits<T>::bytes;
  constexpr int ROWB = StepGeo<T>::ROWB;
  constexpr int BK = ROWB / ES;
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
  constexpr int WGM = WAVES / 2;                     // wave rows; two wave columns
  constexpr int WM = BM / WGM, WN = BN / 2;
  // two waves per SIMD (16-bit types): 16x16x32 MFMA blocks; otherwise 32x32 blocks
  constexpr bool M16 = WAVES == 8 && ES == 2;
  constexpr int BLK = M16 ? 16 : 32;
  constexpr int MI = WM / BLK, NI = WN / BLK;
  static_assert(MI >= 1 && NI >= 1, "tile too small for the wave grid");
  constexpr int A_BYTES = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr int NS = ring_stages(STAGE, BM * BN);
  static_assert(NS >= 2, "the ring needs two stages");
  constexpr bool GATED = EPI == EPI_GATED;
  constexpr int KMMA = M16 ? 32 : (ES == 1 ? 64 : 16);
  constexpr int NSUB = BK / KMMA;
  constexpr int KC = Mma<T>::kChunks;
  static_assert(NSUB % 2 == 0, "fragment double buffer alternates per substep");
  // the MN-major loaders (16-bit, or 8-bit codes)
  using MNA = typename std::conditional<ES == 1, MNTileDma8<BM, WAVES>, MNTileDma<BM, WAVES>>::type;
  static_assert(A_KMAJ || BK == MNA::KROWS, "MN-major stage depth");

  // XA = 1: A has a ring of its own, NSA = NS + 1 stages, and B one of NS (A stages first,
  // then B's); the DMAs of K-step kt+NSA (A) and kt+NS (B) go out in step kt, B's first, so the
  // wait for step kt+1's B leaves the A of step kt+2 in flight
  constexpr int XA = extra_a_stages<T, BM, BN>();
  static_assert(XA == 0 || WAVES == 4, "the extra A stage serves the one-wave-per-SIMD tiles");
  constexpr int NSA = NS + XA;
  constexpr int B_BYTES = BN * ROWB;
  static_assert(NS * STAGE + XA * A_BYTES == dma_ring_bytes<T, BM, BN>(), "ring size");
  auto a_stage = [&](int st) -> char* { return XA ? smem + st * A_BYTES : smem + st * STAGE; };
  auto b_stage = [&](int st) -> char* { return XA ? smem + NSA * A_BYTES + st * B_BYTES : smem + st * STAGE + A_BYTES; };

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int lid = item;
  const int tiles = p.tiles_m * p.tiles_n;
  const int split = lid / tiles;
  lid -= split * tiles;
  int tm, tn;
  grouped_tile(lid, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * (GATED ? BN / 2 : BN);
  const int kbeg = split * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  // ---- DMA loaders. With a K-major A (the DMAs of a K-step go out as one burst after the
  // barrier), an 8-wave tile has its first four waves (one per SIMD) issue every DMA, so the
  // other wave on each SIMD keeps issuing MFMAs while its partner is held up by the burst.
  constexpr int DW = (WAVES == 8 && A_KMAJ) ? 4 : WAVES;
  const bool dma_wave = DW == WAVES || wave < DW;
  KTileDma<T, BM, DW> ka;
  KTileDma<T, BN, DW> kb;
  // offsets per pattern with the burst issue, per instruction when spread (16-bit)
  using NLA = typename std::conditional<ES == 1, MNTileDma8<BM, DW>, MNTileDma<BM, DW, A_KMAJ>>::type;
  using NLB = typename std::conditional<ES == 1, MNTileDma8<BN, DW>, MNTileDma<BN, DW, A_KMAJ>>::type;
  NLA na;
  NLB nb;
  // K-major tile rows: locA / locB(r) -> {base, rows past it} (rows past the matrix clamped)
  const int b_half = BN / 2;
  const int64_t ldb_bytes = (int64_t)p.ldb * ES;
  auto locA = [&](int r) { return make_int2(0, min(m0 + r, p.M - 1) - m0); };
  auto locB = [&](int r) {
    if constexpr (GATED) {   // rows [0, BN/2) from B0 (gate), the rest from B1 (up)
      return r < b_half ? make_int2(0, min(n0 + r, p.N - 1) - n0)
                        : make_int2(1, min(n0 + r - b_half, p.N - 1) - (n0 - b_half));
    } else {                 // rows n >= b_split from B1 when given (stacked [W_gate; W_up])
      const int n = min(n0 + r, p.N - 1);
      return make_int2(p.B1 != nullptr && n >= p.b_split ? 1 : 0, n - n0);
    }
  };
  if constexpr (A_KMAJ) {
    const char* a0 = reinterpret_cast<const char*>(elem_ptr<T>(p.A, m0, p.lda, 0));
    ka.init(lane, kbeg, a0, a0, (int64_t)p.lda * ES, BM, m0 + BM <= p.M);
  } else {
    na.init(wave, lane, reinterpret_cast<const char*>(elem_ptr<T>(p.A, 0, p.lda, m0)), (int64_t)p.lda * ES, kbeg, p.M - m0);
  }
  if constexpr (B_KMAJ) {
    const char* b0 = reinterpret_cast<const char*>(elem_ptr<T>(p.B0, n0, p.ldb, 0));
    if constexpr (GATED) {
      const char* b1 = reinterpret_cast<const char*>(
          reinterpret_cast<uintptr_t>(p.B1) + (int64_t)(n0 - b_half) * ldb_bytes);
      kb.init(lane, kbeg, b0, b1, ldb_bytes, b_half, n0 + b_half <= p.N);
    } else if (p.B1 != nullptr) {
      const char* b1 = reinterpret_cast<const char*>(
          reinterpret_cast<uintptr_t>(p.B1) + (int64_t)(n0 - p.b_split) * ldb_bytes);
      kb.init(lane, kbeg, b0, b1, ldb_bytes, p.b_split - n0, n0 + BN <= p.N);
    } else {
      kb.init(lane, kbeg, b0, b0, ldb_bytes, BN, n0 + BN <= p.N);
    }
  } else {
    nb.init(wave, lane, reinterpret_cast<const char*>(elem_ptr<T>(p.B0, 0, p.ldb, n0)), (int64_t)p.ldb * ES, kbeg, p.N - n0);
  }
  // B stacked from two matrices along K (MN-major only): distance from B0's row k to B1's row
  // k - b_split
  const int64_t b_second = (!B_KMAJ && p.B1 != nullptr)
      ? (reinterpret_cast<const char*>(p.B1) - reinterpret_cast<const char*>(p.B0)) - (int64_t)p.b_split * p.ldb * ES
      : 0;
  const int b_split = (!B_KMAJ && p.B1 != nullptr) ? p.b_split : INT_MAX;
  constexpr int N_DMA = (A_KMAJ ? KTileDma<T, BM, DW>::kInst : NLA::kInst) +
                        (B_KMAJ ? KTileDma<T, BN, DW>::kInst : NLB::kInst);
  constexpr int KIA = A_KMAJ ? KTileDma<T, BM, DW>::kInst : NLA::kInst;
  static_assert((NS - 1) * N_DMA + XA * KIA < 64, "vmcnt range");

  // A / B of K-step kt into A / B ring stage `st`; steps past the end load zeros.
  auto issue_a = [&](int kt, int st) {
    if (!dma_wave) return;
    if constexpr (A_KMAJ) {
      ka.issue(a_stage(st), wave, lane, kt * BK, kend - kbeg, locA);
    } else {
      na.issue(a_stage(st), wave, lane, kbeg + kt * BK, kend, (int64_t)kt * BK * p.lda * ES, INT_MAX, 0);
    }
  };
  auto issue_b = [&](int kt, int st) {
    if (!dma_wave) return;
    if constexpr (B_KMAJ) {
      kb.issue(b_stage(st), wave, lane, kt * BK, kend - kbeg, locB);
    } else {
      nb.issue(b_stage(st), wave, lane, kbeg + kt * BK, kend, (int64_t)kt * BK * p.ldb * ES, b_split, b_second);
    }
  };
  // K-step kt into ring stage `stage` (XA = 0)
  auto issue = [&](int kt, int stage) {
    if (!dma_wave) return;
    issue_a(kt, stage);
    issue_b(kt, stage);
    // the issuing wave is now behind its partner on the SIMD: it wins issue ties until the barrier
    if constexpr (DW < WAVES) __builtin_amdgcn_s_setprio(1);
  };

  // DMA d (0 .. N_DMA-1: A's, then B's) alone: A's of K-step kta into A stage sta, B's of
  // K-step ktb into B stage stb. FAST: the K-step is wholly in range and on one side of
  // b_split, and K-major tiles are interior (the main part of the K loop): scalar bases, no
  // per-lane work
  auto issue_one = [&](int kta, int sta, int ktb, int stb, int d, auto fast) {
    if (!dma_wave) return;
    char* sa = a_stage(sta);
    char* sb = b_stage(stb);
    if constexpr (decltype(fast)::value) {
      if (d < KIA) {
        if constexpr (A_KMAJ) ka.issue_fast_i(sa, wave, d, kta * BK);
        else na.issue_fast_i(sa, wave, d, na.base + (int64_t)kta * BK * p.lda * ES);
      } else {
        if constexpr (B_KMAJ) kb.issue_fast_i(sb, wave, d - KIA, ktb * BK);
        else nb.issue_fast_i(sb, wave, d - KIA,
                             nb.base + (int64_t)ktb * BK * p.ldb * ES + (kbeg + ktb * BK >= b_split ? b_second : 0));
      }
      return;
    }
    if (d < KIA) {
      if constexpr (A_KMAJ) ka.issue_i(sa, wave, lane, d, kta * BK, kend - kbeg, locA);
      else na.issue_i(sa, wave, lane, d, kbeg + kta * BK, kend, (int64_t)kta * BK * p.lda * ES, INT_MAX, 0);
    } else {
      if constexpr (B_KMAJ) kb.issue_i(sb, wave, lane, d - KIA, ktb * BK, kend - kbeg, locB);
      else nb.issue_i(sb, wave, lane, d - KIA, kbeg + ktb * BK, kend, (int64_t)ktb * BK * p.ldb * ES, b_split, b_second);
    }
  };

  // ---- fragment rows / columns of this lane
  const int frow = lane & (BLK - 1), fhalf = lane >> 5, fq = lane >> 4;
  int a_base[MI], b_base[NI];   // first tile row (K-major) / column (MN-major) of each block
#pragma unroll
  for (int i = 0; i < MI; ++i) a_base[i] = wm * WM + i * BLK;   // multiples of 16 (read_block)
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    if constexpr (GATED) {
      constexpr int NH = NI / 2;
      b_base[j] = j < NH ? wn * (WN / 2) + j * BLK : BN / 2 + wn * (WN / 2) + (j - NH) * BLK;
    } else {
      b_base[j] = wn * WN + j * BLK;
    }
  }

  // B fragments single-buffered for the 256-column 16x16 tiles (register budget): B fragment j
  // of the next substep is read right after the last MFMA that uses the current one.
  constexpr bool ROLL = M16 && NI >= 8;
  u32x4 fa[2][MI][KC], fb[ROLL ? 1 : 2][NI][KC];
  auto read_a = [&](int stage, int s, int slot) {
    const char* sa = a_stage(stage);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if constexpr (A_KMAJ && M16) fa[slot][i][c] = KTileDma<T, BM, WAVES>::read_block(sa, a_base[i], frow, 4 * s + fq);
        else if constexpr (A_KMAJ) fa[slot][i][c] = KTileDma<T, BM, WAVES>::read_block(sa, a_base[i], frow, Mma<T>::chunk(s, fhalf, c));
        else if constexpr (M16) fa[slot][i][c] = MNTileDma<BM, WAVES>::read16(sa, a_base[i], s, lane);
        else if constexpr (ES == 1) {
          if (c == 0) MNTileDma8<BM, WAVES>::read8(sa, a_base[i], s, lane, fa[slot][i][0], fa[slot][i][1]);
        } else fa[slot][i][c] = MNTileDma<BM, WAVES>::read(sa, a_base[i], s, lane);
      }
    }
  };
  auto read_b = [&](int stage, int s, int slot, int j) {
    const char* sb = b_stage(stage);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if constexpr (B_KMAJ && M16) fb[slot][j][c] = KTileDma<T, BN, WAVES>::read_block(sb, b_base[j], frow, 4 * s + fq);
      else if constexpr (B_KMAJ) fb[slot][j][c] = KTileDma<T, BN, WAVES>::read_block(sb, b_base[j], frow, Mma<T>::chunk(s, fhalf, c));
      else if constexpr (M16) fb[slot][j][c] = MNTileDma<BN, WAVES>::read16(sb, b_base[j], s, lane);
      else if constexpr (ES == 1) {
        if (c == 0) MNTileDma8<BN, WAVES>::read8(sb, b_base[j], s, lane, fb[slot][j][0], fb[slot][j][1]);
      } else fb[slot][j][c] = MNTileDma<BN, WAVES>::read(sb, b_base[j], s, lane);
    }
  };
  auto read_frags = [&](int stage_a, int stage_b, int s, int slot) {
    read_a(stage_a, s, slot);
#pragma unroll
    for (int j = 0; j < NI; ++j) read_b(stage_b, s, ROLL ? 0 : slot, j);
  };

  using AccV = typename std::conditional<M16, f32x4, f32x16>::type;
  constexpr int ACC_N = M16 ? 4 : 16;
  AccV acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < ACC_N; ++r) acc[i][j][r] = 0.0f;

  constexpr int MN_RD = ES == 1 ? 4 : 2;   // transposing LDS reads per MN-major fragment
  constexpr int N_RD = (A_KMAJ ? MI * KC : MN_RD * MI) + (B_KMAJ ? NI * KC : MN_RD * NI);
  constexpr int N_MMA = MI * NI;

  auto mma_all = [&](int slot) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        if constexpr (M16) Mma16<T>::mma(fb[ROLL ? 0 : slot][j][0], fa[slot][i][0], acc[i][j]);
        else Mma<T>::mma(fb[slot][j], fa[slot][i], acc[i][j]);
      }
  };
  // Where the DMAs of step kt+NS go in the substep after the barrier: with both operands
  // MN-major, spread over the column blocks (every wave issuing its DMAs at once held up the
  // MFMAs queued behind them: dW GEMMs 6-8 % faster spread); with a K-major A, as one burst
  // before the substep's first reads (issuing later made these GEMMs 2-4 % slower).
  constexpr int DMA_COLS = A_KMAJ ? 0 : NI;
  // ROLL: multiply the substep held in fa[slot] / fb, column block by column block, refilling
  // B fragment j with substep s of `stage` as soon as its last MFMA is issued. kt_dma >= 0 and
  // DMA_COLS > 0: also issue the DMAs of K-step kt_dma into stage_dma, spread over the first
  // DMA_COLS column blocks.
  auto mma_roll = [&](int slot, int stage, int s, int kt_dma, int stage_dma, auto fast) {
    if constexpr (ROLL) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
#pragma unroll
        for (int i = 0; i < MI; ++i) Mma16<T>::mma(fb[0][j][0], fa[slot][i][0], acc[i][j]);
        read_b(stage, s, 0, j);
        if constexpr (DMA_COLS > 0) {
          if (kt_dma >= 0 && j < DMA_COLS) {
#pragma unroll
            for (int d = j * N_DMA / DMA_COLS; d < (j + 1) * N_DMA / DMA_COLS; ++d)
              issue_one(kt_dma, stage_dma, kt_dma, stage_dma, d, fast);
          }
        }
      }
    }
  };
  constexpr int RB = B_KMAJ ? KC : MN_RD;         // LDS reads per B fragment
  constexpr int NRA = (A_KMAJ ? KC : MN_RD) * MI;  // LDS reads of the A fragments of a substep

  if (nk > 0) {
    if constexpr (XA) {
      // A of step 0, then (B of step s, A of step s + 1) for s < NS: the order of the loop's
      // issue groups; all but the first group's B and what precedes it may stay in flight.
      // (Written out: as a loop, the compiler took the DMA bases for per-lane values.)
      static_assert(NS == 2, "the extra A stage comes with a two-stage ring");
      issue_a(0, 0);
      issue_b(0, 0);
      issue_a(1, 1);
      issue_b(1, 1);
      issue_a(2, 2);
      wait_vmcnt<KIA + (NS - 1) * N_DMA>();   // step 0 landed
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) issue(s, s);
      wait_vmcnt<(NS - 1) * N_DMA>();   // step 0 landed
    }
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    read_frags(0, 0, 0, 0);
    // drained here so that the loop header's LDS waits are counted from the loop body alone:
    // the prologue issues these reads in another order, and a wait merged over both paths
    // would be lgkmcnt(0) before the first MFMA of every K-step (waiting for the last B
    // fragment refill instead of the first)
    wait_lgkmcnt0();
  }
  // The spread DMA issue (both operands MN-major, or a 4-wave tile) takes the per-lane form
  // only where a step may be partial: the K loop runs as a main part whose DMAs (of step kt+NS)
  // are wholly in range, then the tail.
  using fast_t = std::true_type;
  using slow_t = std::false_type;
  const int nk_full = (kend - kbeg) / BK;
  const bool fast_ok = (!A_KMAJ || ka.interior) && (!B_KMAJ || kb.interior) &&
                       (b_split == INT_MAX || b_split <= kbeg || b_split >= kend || (b_split - kbeg) % BK == 0);
  const int nk_main = fast_ok ? max(0, min(nk, nk_full - NSA)) : 0;
  int cur = 0, cur_a = 0;   // B's (and with XA = 0 A's) ring stage of step kt; A's with XA = 1
  auto k_step = [&](int kt, auto fast) {
    const int nxt = cur + 1 == NS ? 0 : cur + 1;
    const int nxt_a = XA ? (cur_a + 1 == NSA ? 0 : cur_a + 1) : nxt;
    // substeps 0 .. NSUB-2: read substep s+1's fragments while multiplying substep s
#pragma unroll
    for (int s = 0; s + 1 < NSUB; ++s) {
      if constexpr (ROLL) {
        read_a(cur_a, s + 1, (s + 1) & 1);
        mma_roll(s & 1, cur, s + 1, -1, 0, fast);
        interleave_roll<MI, NI, RB, NRA>();
      } else {
        read_frags(cur_a, cur, s + 1, (s + 1) & 1);
        mma_all(s & 1);
        interleave<N_MMA, N_RD, 0>();
      }
    }
    // last substep: step kt+1 must have landed (NS-2 younger steps may be in flight); after
    // the barrier every wave is done reading this stage, which takes step kt+NS
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DW < WAVES) __builtin_amdgcn_s_setprio(0);
    // XA = 1: step kt+1's B went out in the group of step kt+1-NS, before that group's A (of
    // step kt+2) and the NS-2 groups after it; its A went out a group earlier
    wait_vmcnt<(NS - 2) * N_DMA + XA * KIA>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    if constexpr (ROLL) {
      if constexpr (DMA_COLS == 0) issue(kt + NS, cur);
      read_a(nxt_a, 0, 0);
      mma_roll((NSUB - 1) & 1, nxt, 0, kt + NS, cur, fast);
      interleave_roll<MI, NI, RB, NRA>();
    } else {
      if constexpr (WAVES == 4) {
        // one wave per SIMD: a burst would idle the matrix pipe, so the DMAs go one at a time
        // and the interleave pattern places them between the MFMAs
        if constexpr (XA) {
#pragma unroll
          for (int d = KIA; d < N_DMA; ++d) issue_one(0, 0, kt + NS, cur, d, fast);
#pragma unroll
          for (int d = 0; d < KIA; ++d) issue_one(kt + NSA, cur_a, 0, 0, d, fast);
        } else {
#pragma unroll
          for (int d = 0; d < N_DMA; ++d) issue_one(kt + NS, cur, kt + NS, cur, d, fast);
        }
      } else {
        issue(kt + NS, cur);
      }
      read_frags(nxt_a, nxt, 0, 0);
      mma_all((NSUB - 1) & 1);
      interleave<N_MMA, N_RD, N_DMA>();
    }
    cur = nxt;
    cur_a = nxt_a;
  };
  int kt = 0;
  // (not for the 4-wave 256x256 tiles: a second copy of their loop costs them registers)
  if constexpr ((DMA_COLS > 0 && WAVES == 8) || (WAVES == 4 && BM * BN <= 256 * 128)) {
    for (; kt < nk_main; ++kt) k_step(kt, fast_t{});
  }
  for (; kt < nk; ++kt) k_step(kt, slow_t{});
  // the trailing zero-fill DMAs have landed and no wave reads the ring any more: its LDS
  // becomes the epilogue's staging area
  static_assert(epilogue_lds_bytes<BN, WAVES>() <= NS * STAGE, "epilogue staging must fit the ring");
  if constexpr (DW < WAVES) __builtin_amdgcn_s_setprio(0);   // the last issue raised it
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  __builtin_amdgcn_s_barrier();
  epilogue_rows<EPI, IoT, BM, BN, MI, NI, WAVES>(p, acc, m0, n0, split, wm, wn, lane, wave, smem);
}

// One GEMM: a workgroup per tile, placed XCD-aware (xcd_remap).
template <typename T, typename IoT, int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_dma_kernel(const GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[dma_ring_bytes<T, BM, BN>()];
  gemm_dma_tile<T, IoT, BM, BN, A_KMAJ, B_KMAJ, EPI, WAVES>(p, xcd_remap(blockIdx.x, gridDim.x), smem);
}

// Several independent GEMMs in one launch (GemmGroup): member j has the workgroups
// [begin[j], begin[j+1]) and runs the first tile body (kind 0: layout AK0/BK0, epilogue EPI0,
// epilogue type Io0) or the second (kind 1). Each member's range is a multiple of 8 long, so
// xcd_remap keeps its tiles XCD-contiguous; workgroups past a member's tile count do nothing.
// Workgroups are dispatched in index order, so the members listed first start first: listing
// the members with the longest K first lets the short tiles of the others fill the CUs around
// them (list scheduling) instead of each GEMM idling part of the chip in its last round.
template <typename T, int BM, int BN, int WAVES, typename Io0, bool AK0, bool BK0, int EPI0, typename Io1, bool AK1,
          bool BK1, int EPI1>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_dma_group_kernel(const GemmGroup g) {
  __shared__ __attribute__((aligned(1024))) char smem[dma_ring_bytes<T, BM, BN>()];
  const int b = blockIdx.x;
  int j = 0;
  while (j + 1 < g.count && b >= g.begin[j + 1]) ++j;
  const int item = xcd_remap(b - g.begin[j], g.begin[j + 1] - g.begin[j]);
  if (item >= g.items[j]) return;
  if (g.kind[j] == 0) gemm_dma_tile<T, Io0, BM, BN, AK0, BK0, EPI0, WAVES>(g.g[j], item, smem);
  else gemm_dma_tile<T, Io1, BM, BN, AK1, BK1, EPI1, WAVES>(g.g[j], item, smem);
}

template <typename T, int BM, int BN, int WAVES, typename Io0, bool AK0, bool BK0, int EPI0, typename Io1, bool AK1,
          bool BK1, int EPI1>
hipError_t launch_gemm_dma_group(const GemmGroup& g, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_dma_group_kernel<T, BM, BN, WAVES, Io0, AK0, BK0, EPI0, Io1, AK1, BK1, EPI1>),
                     dim3(g.begin[g.count]), dim3(64 * WAVES), 0, stream, g);
  return hipGetLastError();
}

template <typename T, typename IoT, int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI, int WAVES = 4>
hipError_t launch_gemm_dma(const GemmArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_dma_kernel<T, IoT, BM, BN, A_KMAJ, B_KMAJ, EPI, WAVES>), dim3(grid), dim3(64 * WAVES),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace gmlp
