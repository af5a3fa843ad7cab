// Internal declarations shared by the host API and the HIP kernels of librq.
// Citations name the paper "KV Cache Quantization for Looped Transformers with
// 2-Bit Residuals" (ResidualQuant) by section.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "rq.h"

namespace rq {

constexpr int kMaxComp = 8;          // stored components one decode call may read
constexpr int kWaves = 4;            // waves per decode workgroup
constexpr int kThreads = 64 * kWaves;

// Token-pair tile of one wave: G = D/32 lanes cover one token's groups, and a
// lane holds two tokens (t, t + TPW), whose value codes a byte permute pairs in
// one register.
constexpr int groups_of(int D) { return D / 32; }
constexpr int pairs_per_wave(int D) { return 64 / groups_of(D); }
constexpr int tile_tokens(int D) { return 2 * pairs_per_wave(D); }


// Split of the token axis: every (b, h) has nsplit slots. The slot length is
// set on the device from the sequence's own length, so the slots of a ragged
// batch stay balanced: slot_len = unit * ceil(ceil(len / nsplit) / unit), at
// least one unit, where unit is the compressed kernel's wave tile (the BF16
// baseline uses the same slots). nsplit is sized on the host so that the call has about RQ_WGS_PER_CU
// workgroups per compute unit.
struct SplitPlan {
  int unit;
  int nsplit;
};
SplitPlan split_plan(const rq_desc* d);

__host__ __device__ inline int slot_len(int len, int nsplit, int unit) {
  int c = (len + nsplit - 1) / nsplit;
  c = (c + unit - 1) / unit * unit;
  return c < unit ? unit : c;
}

// Slots holding any of the len tokens (slot 0 always counts).
__host__ __device__ inline int slots_used(int len, int nsplit, int unit) {
  if (len <= 0) return 1;
  const int c = slot_len(len, nsplit, unit);
  return (len + c - 1) / c;
}

constexpr size_t part_floats(int D) { return (size_t)D + 4; }

// Workspace: B*H*nsplit partials of D+4 floats (m, l, -, -, acc[D]).

// What the combine needs to produce the output from the partials.
struct CombineParams {
  const float* part;        // split partials
  const int32_t* past_len;  // device [B]
  const uint16_t* q;        // bf16 [B][H][D]
  const uint16_t* kcur;     // bf16 [B][H][D]
  const uint16_t* vcur;     // bf16 [B][H][D]
  const void* rotv;         // [H][D][D] (fp32, or fp16 if rot_f16), or nullptr (no value rotation)
  float* out;               // fp32 [B][H][D]
  int32_t* dev_err;
  float scale_log2;         // softmax scale * log2(e)
  int B, H, T_max, unit, nsplit;
  int rot_f16;              // rotv holds fp16 entries
};

struct DecodeParams {
  const uint8_t* kcodes[kMaxComp];
  const uint32_t* kmeta[kMaxComp];
  const uint16_t* kalpha[kMaxComp];   // [c] for c >= 1: alpha linking component c-1 to c
  const uint8_t* vcodes[kMaxComp];
  const uint32_t* vmeta[kMaxComp];
  const uint16_t* valpha[kMaxComp];
  const void* rotk;                   // [H][D][D], fp32 (or fp16 if rot_f16)
  const uint16_t* q;                  // bf16 [B][H][D]
  const int32_t* past_len;
  float* part;
  float scale_log2;
  int B, H, T_max, unit, nsplit;
  int rot_f16;                        // rotk holds fp16 entries
  // paged cache (table == nullptr: contiguous): block table [B][maxblk], block
  // size 2^lbs tokens, pool of num_blocks blocks = pool_rows rows per buffer
  const int32_t* table;
  int maxblk, lbs, num_blocks;
  uint32_t pool_rows;
  int32_t* dev_err;                   // may be null
};

struct Bf16Params {
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q;
  const int32_t* past_len;
  float* part;
  float scale_log2;
  int B, H, T_max, unit, nsplit;
};

struct AppendParams {
  uint8_t* codes[2][RQ_MAX_LOOPS];
  uint32_t* meta[2][RQ_MAX_LOOPS];
  uint16_t* alpha[2][RQ_MAX_LOOPS];
  const void* rot[2];       // [H][D][D] per tensor, fp32 (or fp16 if rot_f16)
  const uint16_t* kv;       // bf16 [2][L][B][H][n][D]
  const int32_t* pos;
  int32_t* dev_err;
  int B, H, L, n, T_max, policy;
  int G;                    // loops per anchor group (divides L)
  uint32_t g16;             // bit r: loop r is INT2 in groups of 16 channels (else groups of 32)
  const int32_t* table;     // paged cache: block table [B][maxblk], blocks of 2^lbs tokens; else null
  int maxblk, lbs, num_blocks;
  int rot_f16;              // the rotations hold fp16 entries
  int bits[RQ_MAX_LOOPS];
};

// One-token (or few-token) appends, one workgroup per (token, head, tensor,
// layer). The cache pointers of the launch's layers travel in the kernel
// arguments, so one launch serves many layers without a table in device memory:
// layer i's pointers start at slot i * stride, as
//   [block table, then per tensor (K, V): rotation, codes[0..L-1], meta[0..L-1],
//    alpha[0..L-1]], stride = 1 + 2 (1 + 3 L).
// kUnitSlots keeps the whole argument block below 4 KB.
constexpr int kUnitSlots = 440;
constexpr int unit_stride(int L) { return 1 + 2 * (1 + 3 * L); }
struct UnitParams {
  const uint16_t* kv;       // bf16 [nl][2][L][B][H][n][D]
  const int32_t* pos;
  int32_t* dev_err;
  int B, H, L, n, T_max, policy;
  int G;                    // loops per anchor group (divides L)
  uint32_t g16;             // bit r: loop r is INT2 in groups of 16 channels
  int maxblk, lbs, num_blocks;  // paged cache (block size 2^lbs); maxblk = 0: contiguous
  int nl;                   // layers in this launch
  int upw;                  // (sequence, token) units per workgroup
  int rot_f16;              // the rotations (slot per tensor) hold fp16 entries
  int bits[RQ_MAX_LOOPS];
  const void* slot[kUnitSlots];
};
static_assert(sizeof(UnitParams) <= 4096, "kernel arguments must stay within 4 KB");

struct PrefillParams {
  const uint16_t* q;        // bf16 [B][H][T][D]
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* lens;      // [B], clamped to [0, T]
  float* out;               // fp32 [B][H][T][D]
  uint16_t* vt;             // workspace: fp16 V^T [B][H][D][Tp]
  int32_t* dev_err;         // may be null
  float scale_log2;
  int B, H, T, Tp;          // Tp: T rounded up to the key tile
};

// Launchers (return hipError_t as int; 0 = success). Defined in the .hip files.
int launch_append(const AppendParams& p, int D, void* stream);
// n <= kUnitAppendMax tokens per sequence, or more than 16 loops.
constexpr int kUnitAppendMax = 8;
int launch_append_unit(const UnitParams& p, int D, void* stream);
// ncomp components of kinds bits[0..ncomp-1], the rotated query in `limbs` 7-bit
// limbs (2 or 3); returns -1 if no kernel exists.
int launch_decode(const DecodeParams& p, int D, int ncomp, const int* bits, int limbs, int nsplit, void* stream);
int launch_decode_paged(const DecodeParams& p, int D, int ncomp, const int* bits, int limbs, int nsplit,
                        void* stream);
int launch_bf16(const Bf16Params& p, int D, int nsplit, void* stream);
// cols: output columns per workgroup, 32 or D
int launch_combine(const CombineParams& p, int D, int cols, void* stream);
int launch_prefill(const PrefillParams& p, int D, void* stream);
size_t prefill_workspace_bytes(int B, int H, int D, int T);
// paged: a paged cache (chains of more than four components have contiguous instances only)
bool have_decode_kernel(int D, int ncomp, const int* bits, int limbs, bool paged);
bool have_decode_kernel_long(int D, int ncomp, const int* bits, int limbs);
int launch_decode_long(const DecodeParams& p, int D, int ncomp, const int* bits, int limbs, int nsplit,
                       void* stream);

}  // namespace rq
