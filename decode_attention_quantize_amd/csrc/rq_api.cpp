// Host side of librq: argument validation, buffer sizes, split planning and
// kernel dispatch for the C ABI declared in include/rq.h.
#include <cmath>
#include <cstring>
#include <mutex>

#include <hip/hip_runtime.h>

#include "rq_internal.hpp"

namespace rq {

// Compute units of the current device (the workspace size depends on it).
static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return cus;
}

#ifndef RQ_WGS_PER_CU
#define RQ_WGS_PER_CU 3
#endif

#ifndef RQ_MIN_SLOT_TILES
#define RQ_MIN_SLOT_TILES 8
#endif

SplitPlan split_plan(const rq_desc* d) {
  // About RQ_WGS_PER_CU workgroups per compute unit over the whole call, but
  // no more slots than leave each at least RQ_MIN_SLOT_TILES tiles of the
  // cache's capacity: a workgroup's fixed work (the query rotation, its partial)
  // costs about as much as streaming that many tiles. Where rounding the slot
  // count up would overshoot that target (some workgroups would wait for a
  // second round), two workgroups per compute unit, each with longer slots,
  // measured faster (B4 H55 D96 at 4096 tokens: 4 slots -> 2, 3-9 % per call).
  // Slot lengths are set per sequence on the device (slot_len).
  const long long unit = tile_tokens(d->head_dim);
  const long long bh = (long long)d->batch * d->heads;
  const long long target = (long long)RQ_WGS_PER_CU * device_cus();
  long long nsplit = (target + bh - 1) / bh;
  if (nsplit * bh > target) nsplit = 2LL * device_cus() / bh;
  if (nsplit < 1) nsplit = 1;
  const long long cap = d->max_tokens / (unit * RQ_MIN_SLOT_TILES);
  if (nsplit > cap) nsplit = cap;
  if (nsplit < 1) nsplit = 1;
  SplitPlan p;
  p.unit = (int)unit;
  p.nsplit = (int)nsplit;
  return p;
}

}  // namespace rq

using namespace rq;

namespace {

bool dim_ok(int D) { return D == 64 || D == 96 || D == 128; }

constexpr float kLog2e = 1.4426950408889634f;

bool al(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int log2_of(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

rq_status check_shape(const rq_desc* d) {
  if (!d) return RQ_E_NULL;
  if (d->batch < 1 || d->heads < 1 || !dim_ok(d->head_dim) || d->loops < 1 || d->loops > RQ_MAX_LOOPS ||
      d->max_tokens < 1 || (d->flags & ~(RQ_FLAG_PRECISE_QUERY | RQ_FLAG_ROT_F16)) != 0)
    return RQ_E_SHAPE;
  return RQ_OK;
}

rq_status check_plan(const rq_desc* d) {
  rq_status s = check_shape(d);
  if (s != RQ_OK) return s;
  if (d->policy != RQ_POLICY_LAST_LOOP && d->policy != RQ_POLICY_PREV_LOOP && d->policy != RQ_POLICY_FIRST_LOOP)
    return RQ_E_POLICY;
  if (d->loop_group < 0 || d->loop_group > d->loops || (d->loop_group > 0 && d->loops % d->loop_group != 0))
    return RQ_E_SHAPE;
  if (d->block_size != 0) {  // paged cache
    const int bs = d->block_size;
    if (bs < 16 || bs > 4096 || (bs & (bs - 1)) != 0 || d->max_tokens % bs != 0 || d->num_blocks < 1)
      return RQ_E_SHAPE;
    // every pool buffer (the largest: INT4 codes, D/2 bytes per row) stays addressable by
    // the 32-bit offsets of the decode kernel's buffer loads
    const uint64_t rows = (uint64_t)d->num_blocks * (uint64_t)d->heads * (uint64_t)bs;
    if (rows * (uint64_t)(d->head_dim / 2) > 0xFFFF0000ull) return RQ_E_SHAPE;
  }
  for (int r = 0; r < d->loops; ++r) {
    if (d->bits[r] != 2 && d->bits[r] != 4) return RQ_E_BITS;
    if (d->group[r] != 32 && !(d->group[r] == 16 && d->bits[r] == 2)) return RQ_E_BITS;
  }
  return RQ_OK;
}

// Loops per anchor group (loop_group 0 = one group of all loops).
int group_len(const rq_desc* d) { return d->loop_group > 0 ? d->loop_group : d->loops; }

// Anchor of the group holding loop r (0-based): its last loop under Last-loop,
// its first under First-loop and Previous-loop (§3.2; §5 "Models").
int anchor_of(const rq_desc* d, int r) {
  const int G = group_len(d), g0 = r / G * G;
  return d->policy == RQ_POLICY_LAST_LOOP ? g0 + G - 1 : g0;
}

size_t workspace_for(const rq_desc* d) {
  const SplitPlan sp = split_plan(d);
  const size_t bh = (size_t)d->batch * d->heads;
  return bh * sp.nsplit * part_floats(d->head_dim) * 4;
}

CombineParams combine_params(const rq_desc* d, void* ws, const uint16_t* q, const uint16_t* k_cur,
                             const uint16_t* v_cur, const int32_t* past_len, const void* rotv, float* out,
                             int32_t* dev_err, float scale_log2) {
  const SplitPlan sp = split_plan(d);
  CombineParams a;
  a.part = static_cast<float*>(ws);
  a.past_len = past_len;
  a.q = q;
  a.kcur = k_cur;
  a.vcur = v_cur;
  a.rotv = rotv;
  a.out = out;
  a.dev_err = dev_err;
  a.scale_log2 = scale_log2;
  a.B = d->batch;
  a.H = d->heads;
  a.T_max = d->max_tokens;
  a.unit = sp.unit;
  a.nsplit = sp.nsplit;
  a.rot_f16 = (d->flags & RQ_FLAG_ROT_F16) ? 1 : 0;
  return a;
}

// Components decode loop r reads, anchor first (§3.2, App. D): the shared
// anchor and r itself, or the chain from the group's first loop up to r.
int components(const rq_desc* d, int r, int* loops) {
  const int a = anchor_of(d, r);
  if (d->policy != RQ_POLICY_PREV_LOOP) {
    loops[0] = a;
    if (r == a) return 1;
    loops[1] = r;
    return 2;
  }
  for (int c = a; c <= r; ++c) loops[c - a] = c;
  return r - a + 1;
}

}  // namespace

extern "C" {

const char* rq_status_str(rq_status s) {
  switch (s) {
    case RQ_OK: return "ok";
    case RQ_E_NULL: return "required pointer is NULL";
    case RQ_E_SHAPE: return "shape out of range (batch, heads, head_dim in {64,96,128}, loops 1..32, loop_group 0 or a divisor of loops, max_tokens >= 1, n, known flags)";
    case RQ_E_BITS: return "unsupported bit width or group size (bits 2 or 4; group 32, or 16 for 2 bits)";
    case RQ_E_CAPACITY: return "size exceeds max_tokens";
    case RQ_E_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case RQ_E_UNSUPPORTED: return "no kernel for this combination (e.g. a chain of more than 8 components, or of more than 4 in a paged cache)";
    case RQ_E_HIP: return "HIP launch failed";
    case RQ_E_POLICY: return "unknown reference policy";
    case RQ_E_LOOP: return "loop index out of range";
    case RQ_E_ALIGN: return "device array misaligned (codes/rot/kv/q/k/v 16 B, meta 4 B (8 B for groups of 16), out 4 B, alpha 2 B)";
    case RQ_E_SCRATCH: return "the call's split partials exceed the library's static scratch (RQ_SCRATCH_BYTES); use rq_decode_attn with a workspace";
  }
  return "unknown status";
}

const char* rq_version(void) { return "rq 0.1 (gfx950)"; }

rq_status rq_check_desc(const rq_desc* d) { return check_plan(d); }

size_t rq_buffer_bytes(const rq_desc* d, int kind, int loop) {
  if (check_plan(d) != RQ_OK || loop < 0 || loop >= d->loops) return 0;
  const size_t toks = d->block_size ? (size_t)d->num_blocks * d->heads * d->block_size
                                    : (size_t)d->batch * d->heads * d->max_tokens;
  switch (kind) {
    case 0: return toks * d->head_dim * d->bits[loop] / 8;
    case 1: return toks * (d->head_dim / d->group[loop]) * 4;
    case 2: return toks * 2;
  }
  return 0;
}

size_t rq_workspace_bytes(const rq_desc* d) {
  if (check_shape(d) != RQ_OK) return 0;
  return workspace_for(d);
}

}  // extern "C"

namespace {

// Pointer and alignment checks of one layer's cache for an append.
rq_status check_append_cache(const rq_desc* d, const rq_layer_cache* c) {
  if (!c->rot[0] || !c->rot[1]) return RQ_E_NULL;
  if (!al(c->rot[0], 16) || !al(c->rot[1], 16)) return RQ_E_ALIGN;
  for (int kvi = 0; kvi < 2; ++kvi) {
    for (int r = 0; r < d->loops; ++r) {
      if (!c->codes[kvi][r] || !c->meta[kvi][r]) return RQ_E_NULL;
      const bool anchor = r == anchor_of(d, r);
      if (!anchor && !c->alpha[kvi][r]) return RQ_E_NULL;
      const uintptr_t ma = d->group[r] == 16 ? 8 : 4;
      if (!al(c->codes[kvi][r], 16) || !al(c->meta[kvi][r], ma) || (!anchor && !al(c->alpha[kvi][r], 2)))
        return RQ_E_ALIGN;
    }
  }
  if (d->block_size) {
    if (!c->block_table) return RQ_E_NULL;
    if (!al(c->block_table, 4)) return RQ_E_ALIGN;
  }
  return RQ_OK;
}

// Appends n tokens to nl layers (caches[0..nl-1]); kv holds the layers' inputs
// back to back. Every check runs before the first launch.
rq_status append_layers(const rq_desc* d, const rq_layer_cache* caches, int32_t nl, const uint16_t* kv,
                        const int32_t* pos, int32_t n, int32_t* dev_err, void* stream) {
  rq_status s = check_plan(d);
  if (s != RQ_OK) return s;
  if (!caches) return RQ_E_NULL;
  if (n < 0 || nl < 0) return RQ_E_SHAPE;
  if (n > d->max_tokens) return RQ_E_CAPACITY;
  if (n == 0 || nl == 0) return RQ_OK;
  if (!kv || !pos) return RQ_E_NULL;
  if (!al(kv, 16) || !al(pos, 4)) return RQ_E_ALIGN;
  for (int l = 0; l < nl; ++l)
    if ((s = check_append_cache(d, &caches[l])) != RQ_OK) return s;
  const size_t layer_elems = (size_t)2 * d->loops * d->batch * d->heads * n * d->head_dim;
  const int lbs = d->block_size ? log2_of(d->block_size) : 0;
  const int maxblk = d->block_size ? d->max_tokens / d->block_size : 0;
  uint32_t g16 = 0;
  for (int r = 0; r < d->loops; ++r)
    if (d->group[r] == 16) g16 |= 1u << r;

  if (n <= kUnitAppendMax || d->loops > 16) {
    // per-unit kernel, as many layers per launch as the argument slots hold
    UnitParams p;
    std::memset(&p, 0, sizeof(p));
    p.pos = pos;
    p.dev_err = dev_err;
    p.B = d->batch;
    p.H = d->heads;
    p.L = d->loops;
    p.n = n;
    p.T_max = d->max_tokens;
    p.policy = d->policy;
    p.G = group_len(d);
    p.g16 = g16;
    p.maxblk = maxblk;
    p.lbs = lbs;
    p.num_blocks = d->num_blocks;
    p.rot_f16 = (d->flags & RQ_FLAG_ROT_F16) ? 1 : 0;
    for (int r = 0; r < d->loops; ++r) p.bits[r] = d->bits[r];
    const int stride = unit_stride(d->loops);
    const int per = kUnitSlots / stride;
    for (int l0 = 0; l0 < nl; l0 += per) {
      p.nl = nl - l0 < per ? nl - l0 : per;
      // Units share a workgroup (and its staging of the rotation) while that
      // still leaves about two workgroups per compute unit.
      const long long units = (long long)d->batch * n;
      long long upw = units * d->heads * 2 * p.nl / (2LL * device_cus());
      if (upw < 1) upw = 1;
      if (upw > units) upw = units;
      const long long runs = (units + upw - 1) / upw;
      p.upw = (int)((units + runs - 1) / runs);
      p.kv = kv + (size_t)l0 * layer_elems;
      for (int i = 0; i < p.nl; ++i) {
        const rq_layer_cache* c = &caches[l0 + i];
        const void** sl = p.slot + (size_t)i * stride;
        sl[0] = d->block_size ? c->block_table : nullptr;
        for (int kvi = 0; kvi < 2; ++kvi) {
          const void** st = sl + 1 + kvi * (1 + 3 * d->loops);
          st[0] = c->rot[kvi];
          for (int r = 0; r < d->loops; ++r) {
            st[1 + r] = c->codes[kvi][r];
            st[1 + d->loops + r] = c->meta[kvi][r];
            st[1 + 2 * d->loops + r] = c->alpha[kvi][r];
          }
        }
      }
      if (launch_append_unit(p, d->head_dim, stream) != 0) return RQ_E_HIP;
    }
    return RQ_OK;
  }

  // bulk kernel (fp64 matrix cores), one launch per layer
  for (int l = 0; l < nl; ++l) {
    const rq_layer_cache* c = &caches[l];
    AppendParams p;
    std::memset(&p, 0, sizeof(p));
    for (int kvi = 0; kvi < 2; ++kvi) {
      for (int r = 0; r < d->loops; ++r) {
        p.codes[kvi][r] = c->codes[kvi][r];
        p.meta[kvi][r] = reinterpret_cast<uint32_t*>(c->meta[kvi][r]);
        p.alpha[kvi][r] = c->alpha[kvi][r];
      }
      p.rot[kvi] = c->rot[kvi];
    }
    p.kv = kv + (size_t)l * layer_elems;
    p.pos = pos;
    p.dev_err = dev_err;
    p.B = d->batch;
    p.H = d->heads;
    p.L = d->loops;
    p.n = n;
    p.T_max = d->max_tokens;
    p.policy = d->policy;
    p.G = group_len(d);
    p.g16 = g16;
    p.rot_f16 = (d->flags & RQ_FLAG_ROT_F16) ? 1 : 0;
    if (d->block_size) {
      p.table = c->block_table;
      p.maxblk = maxblk;
      p.lbs = lbs;
      p.num_blocks = d->num_blocks;
    }
    for (int r = 0; r < d->loops; ++r) p.bits[r] = d->bits[r];
    if (launch_append(p, d->head_dim, stream) != 0) return RQ_E_HIP;
  }
  return RQ_OK;
}

}  // namespace

extern "C" {

rq_status rq_quantize_append(const rq_desc* d, const rq_layer_cache* c, const uint16_t* kv,
                             const int32_t* pos, int32_t n, int32_t* dev_err, void* stream) {
  return append_layers(d, c, 1, kv, pos, n, dev_err, stream);
}

rq_status rq_quantize_append_layers(const rq_desc* d, const rq_layer_cache* caches, int32_t nlayers,
                                    const uint16_t* kv, const int32_t* pos, int32_t n, int32_t* dev_err,
                                    void* stream) {
  return append_layers(d, caches, nlayers, kv, pos, n, dev_err, stream);
}

rq_status rq_split_plan(const rq_desc* d, int32_t* unit, int32_t* nsplit) {
  const rq_status s = check_shape(d);
  if (s != RQ_OK) return s;
  if (!unit || !nsplit) return RQ_E_NULL;
  const SplitPlan sp = split_plan(d);
  *unit = sp.unit;
  *nsplit = sp.nsplit;
  return RQ_OK;
}

}  // extern "C"

namespace {

// Whether a streaming kernel exists for the components decode of `loop` reads
// under d (their kinds, the head size, the query precision, the cache mode).
bool decode_supported(const rq_desc* d, int32_t loop) {
  int loops[RQ_MAX_LOOPS];
  const int nc = components(d, loop, loops);
  if (nc > kMaxComp) return false;
  int kinds[kMaxComp];
  for (int i = 0; i < nc; ++i) kinds[i] = d->bits[loops[i]] | (d->group[loops[i]] == 16 ? 8 : 0);
  const int limbs = (d->flags & RQ_FLAG_PRECISE_QUERY) ? 3 : 2;
  return have_decode_kernel(d->head_dim, nc, kinds, limbs, d->block_size != 0);
}

rq_status decode_partial(const rq_desc* d, const rq_layer_cache* c, int32_t loop, const uint16_t* q,
                         const int32_t* past_len, float softmax_scale, void* ws, size_t ws_bytes, int32_t* dev_err,
                         void* stream) {
  rq_status s = check_plan(d);
  if (s != RQ_OK) return s;
  if (!c) return RQ_E_NULL;
  if (loop < 0 || loop >= d->loops) return RQ_E_LOOP;
  if (!q || !past_len || !c->rot[0]) return RQ_E_NULL;
  if (!al(q, 16) || !al(past_len, 4) || !al(c->rot[0], 16)) return RQ_E_ALIGN;
  if (!ws || ws_bytes < workspace_for(d) || ((uintptr_t)ws & 255) != 0) return RQ_E_WORKSPACE;
  if (!std::isfinite(softmax_scale)) return RQ_E_SHAPE;
  int loops[RQ_MAX_LOOPS];
  const int nc = components(d, loop, loops);
  int bits[kMaxComp];  // component kinds: bit width, plus 8 for INT2 in groups of 16
  const int limbs = (d->flags & RQ_FLAG_PRECISE_QUERY) ? 3 : 2;
  if (!decode_supported(d, loop)) return RQ_E_UNSUPPORTED;
  for (int i = 0; i < nc; ++i) bits[i] = d->bits[loops[i]] | (d->group[loops[i]] == 16 ? 8 : 0);

  const SplitPlan sp = split_plan(d);
  DecodeParams p;
  std::memset(&p, 0, sizeof(p));
  for (int i = 0; i < nc; ++i) {
    const int r = loops[i];
    if (!c->codes[0][r] || !c->meta[0][r] || !c->codes[1][r] || !c->meta[1][r]) return RQ_E_NULL;
    const uintptr_t ma = d->group[r] == 16 ? 8 : 4;  // metadata of a 32-channel block: 4 or 8 bytes
    if (!al(c->codes[0][r], 16) || !al(c->codes[1][r], 16) || !al(c->meta[0][r], ma) || !al(c->meta[1][r], ma))
      return RQ_E_ALIGN;
    p.kcodes[i] = c->codes[0][r];
    p.kmeta[i] = reinterpret_cast<const uint32_t*>(c->meta[0][r]);
    p.vcodes[i] = c->codes[1][r];
    p.vmeta[i] = reinterpret_cast<const uint32_t*>(c->meta[1][r]);
    if (i > 0) {
      if (!c->alpha[0][r] || !c->alpha[1][r]) return RQ_E_NULL;
      if (!al(c->alpha[0][r], 2) || !al(c->alpha[1][r], 2)) return RQ_E_ALIGN;
      p.kalpha[i] = c->alpha[0][r];
      p.valpha[i] = c->alpha[1][r];
    }
  }
  p.rotk = c->rot[0];
  p.rot_f16 = (d->flags & RQ_FLAG_ROT_F16) ? 1 : 0;
  p.q = q;
  p.past_len = past_len;
  p.part = static_cast<float*>(ws);
  p.scale_log2 = softmax_scale * kLog2e;
  p.B = d->batch;
  p.H = d->heads;
  p.T_max = d->max_tokens;
  p.unit = sp.unit;
  p.nsplit = sp.nsplit;
  p.dev_err = dev_err;
  if (d->block_size) {
    if (!c->block_table) return RQ_E_NULL;
    if (!al(c->block_table, 4)) return RQ_E_ALIGN;
    p.table = c->block_table;
    p.maxblk = d->max_tokens / d->block_size;
    p.lbs = log2_of(d->block_size);
    p.num_blocks = d->num_blocks;
    p.pool_rows = (uint32_t)((size_t)d->num_blocks * d->heads * d->block_size);
  }
  return launch_decode(p, d->head_dim, nc, bits, limbs, sp.nsplit, stream) == 0 ? RQ_OK : RQ_E_HIP;
}

}  // namespace

extern "C" {

rq_status rq_check_decode(const rq_desc* d, int32_t loop) {
  const rq_status s = check_plan(d);
  if (s != RQ_OK) return s;
  if (loop < 0 || loop >= d->loops) return RQ_E_LOOP;
  return decode_supported(d, loop) ? RQ_OK : RQ_E_UNSUPPORTED;
}

rq_status rq_decode_attn_partial(const rq_desc* d, const rq_layer_cache* c, int32_t loop, const uint16_t* q,
                                 const int32_t* past_len, float softmax_scale, void* ws, size_t ws_bytes,
                                 void* stream) {
  return decode_partial(d, c, loop, q, past_len, softmax_scale, ws, ws_bytes, nullptr, stream);
}

rq_status rq_decode_combine(const rq_desc* d, const void* rot_v, const uint16_t* q, const uint16_t* k_cur,
                            const uint16_t* v_cur, const int32_t* past_len, float softmax_scale, float* out,
                            const void* ws, size_t ws_bytes, int32_t* dev_err, void* stream) {
  rq_status s = check_shape(d);
  if (s != RQ_OK) return s;
  if (!q || !k_cur || !v_cur || !past_len || !out) return RQ_E_NULL;
  if (!al(q, 16) || !al(k_cur, 16) || !al(v_cur, 16) || !al(past_len, 4) || !al(out, 4) ||
      (rot_v && !al(rot_v, 16)))
    return RQ_E_ALIGN;
  if (!ws || ws_bytes < workspace_for(d) || ((uintptr_t)ws & 255) != 0) return RQ_E_WORKSPACE;
  if (!std::isfinite(softmax_scale)) return RQ_E_SHAPE;
  const CombineParams cp = combine_params(d, const_cast<void*>(ws), q, k_cur, v_cur, past_len, rot_v, out,
                                          dev_err, softmax_scale * kLog2e);
  // the value rotation's product spread over D/32 workgroups per (b, h) while
  // that leaves no more workgroups than compute units, else (D = 128) over two
  // while that does (B8 H16: 256 workgroups, 4.3 against 4.6 us per call)
  const long long narrow = (long long)d->batch * d->heads * (d->head_dim / 32);
  const int cols = (rot_v && narrow <= device_cus()) ? 32
                   : (rot_v && d->head_dim == 128 && narrow / 2 <= device_cus()) ? 64 : d->head_dim;
  return launch_combine(cp, d->head_dim, cols, stream) == 0 ? RQ_OK : RQ_E_HIP;
}

}  // extern "C"

namespace {

// Checks of a whole decode call that come before its workspace.
rq_status check_decode_call(const rq_desc* d, const rq_layer_cache* c, int32_t loop, const uint16_t* q,
                            const uint16_t* k_cur, const uint16_t* v_cur, const int32_t* past_len, const float* out) {
  rq_status s = check_plan(d);
  if (s != RQ_OK) return s;
  if (!c) return RQ_E_NULL;
  if (loop < 0 || loop >= d->loops) return RQ_E_LOOP;
  if (!q || !k_cur || !v_cur || !past_len || !out || !c->rot[0] || !c->rot[1]) return RQ_E_NULL;
  if (!al(q, 16) || !al(k_cur, 16) || !al(v_cur, 16) || !al(past_len, 4) || !al(out, 4) || !al(c->rot[0], 16) ||
      !al(c->rot[1], 16))
    return RQ_E_ALIGN;
  return RQ_OK;
}

}  // namespace

extern "C" {

rq_status rq_decode_attn(const rq_desc* d, const rq_layer_cache* c, int32_t loop, const uint16_t* q,
                         const uint16_t* k_cur, const uint16_t* v_cur, const int32_t* past_len,
                         float softmax_scale, float* out, void* ws, size_t ws_bytes, int32_t* dev_err,
                         void* stream) {
  rq_status s = check_decode_call(d, c, loop, q, k_cur, v_cur, past_len, out);
  if (s != RQ_OK) return s;
  // Validate everything the second launch needs before enqueuing the first.
  if (!ws || ws_bytes < workspace_for(d) || ((uintptr_t)ws & 255) != 0) return RQ_E_WORKSPACE;
  s = decode_partial(d, c, loop, q, past_len, softmax_scale, ws, ws_bytes, dev_err, stream);
  if (s != RQ_OK) return s;
  return rq_decode_combine(d, c->rot[1], q, k_cur, v_cur, past_len, softmax_scale, out, ws, ws_bytes, dev_err,
                           stream);
}

}  // extern "C"

// ---- decode without a caller workspace -------------------------------------
// The split partials live in a file-scope device array instead: every GPU the
// library runs on holds its own copy for the life of the process, and its
// address on each device is looked up once, with that device current.
static __device__ __align__(256) unsigned char scratch[RQ_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Address of the current device's scratch (nullptr if it cannot be found).
void* scratch_of_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}
}  // namespace

extern "C" {

rq_status rq_decode_attn_noalloc(const rq_desc* d, const rq_layer_cache* c, int32_t loop, const uint16_t* q,
                                 const uint16_t* k_cur, const uint16_t* v_cur, const int32_t* past_len,
                                 float softmax_scale, float* out, int32_t* dev_err, void* stream) {
  const rq_status s = check_decode_call(d, c, loop, q, k_cur, v_cur, past_len, out);
  if (s != RQ_OK) return s;
  if (workspace_for(d) > (size_t)RQ_SCRATCH_BYTES) return RQ_E_SCRATCH;
  void* ws = scratch_of_current_device();
  if (!ws) return RQ_E_HIP;
  return rq_decode_attn(d, c, loop, q, k_cur, v_cur, past_len, softmax_scale, out, ws, (size_t)RQ_SCRATCH_BYTES,
                        dev_err, stream);
}

rq_status rq_decode_attn_bf16_partial(const rq_desc* d, const uint16_t* k_cache, const uint16_t* v_cache,
                                      const uint16_t* q, const int32_t* past_len, float softmax_scale, void* ws,
                                      size_t ws_bytes, void* stream) {
  rq_status s = check_shape(d);
  if (s != RQ_OK) return s;
  if (!k_cache || !v_cache || !q || !past_len) return RQ_E_NULL;
  if (!al(k_cache, 16) || !al(v_cache, 16) || !al(q, 16) || !al(past_len, 4)) return RQ_E_ALIGN;
  if (!ws || ws_bytes < workspace_for(d) || ((uintptr_t)ws & 255) != 0) return RQ_E_WORKSPACE;
  if (!std::isfinite(softmax_scale)) return RQ_E_SHAPE;
  const SplitPlan sp = split_plan(d);
  Bf16Params p;
  p.k = k_cache;
  p.v = v_cache;
  p.q = q;
  p.past_len = past_len;
  p.part = static_cast<float*>(ws);
  p.scale_log2 = softmax_scale * kLog2e;
  p.B = d->batch;
  p.H = d->heads;
  p.T_max = d->max_tokens;
  p.unit = sp.unit;
  p.nsplit = sp.nsplit;
  return launch_bf16(p, d->head_dim, sp.nsplit, stream) == 0 ? RQ_OK : RQ_E_HIP;
}

rq_status rq_decode_attn_bf16(const rq_desc* d, const uint16_t* k_cache, const uint16_t* v_cache,
                              const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                              const int32_t* past_len, float softmax_scale, float* out, void* ws,
                              size_t ws_bytes, int32_t* dev_err, void* stream) {
  rq_status s = check_shape(d);
  if (s != RQ_OK) return s;
  if (!k_cache || !v_cache || !q || !k_cur || !v_cur || !past_len || !out) return RQ_E_NULL;
  if (!al(k_cache, 16) || !al(v_cache, 16) || !al(q, 16) || !al(k_cur, 16) || !al(v_cur, 16) ||
      !al(past_len, 4) || !al(out, 4))
    return RQ_E_ALIGN;
  if (!ws || ws_bytes < workspace_for(d) || ((uintptr_t)ws & 255) != 0) return RQ_E_WORKSPACE;
  if (!std::isfinite(softmax_scale)) return RQ_E_SHAPE;
  s = rq_decode_attn_bf16_partial(d, k_cache, v_cache, q, past_len, softmax_scale, ws, ws_bytes, stream);
  if (s != RQ_OK) return s;
  return rq_decode_combine(d, nullptr, q, k_cur, v_cur, past_len, softmax_scale, out, ws, ws_bytes, dev_err, stream);
}

size_t rq_prefill_workspace_bytes(const rq_desc* d, int32_t n) {
  if (check_shape(d) != RQ_OK || n < 0) return 0;
  return prefill_workspace_bytes(d->batch, d->heads, d->head_dim, n);
}

rq_status rq_prefill_attn(const rq_desc* d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const int32_t* lens, int32_t n, float softmax_scale, float* out, void* ws,
                          size_t ws_bytes, int32_t* dev_err, void* stream) {
  rq_status s = check_shape(d);
  if (s != RQ_OK) return s;
  if (n < 0) return RQ_E_SHAPE;
  if (n == 0) return RQ_OK;
  if (!q || !k || !v || !lens || !out) return RQ_E_NULL;
  if (!al(q, 16) || !al(k, 16) || !al(v, 16) || !al(out, 16) || !al(lens, 4)) return RQ_E_ALIGN;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f)) return RQ_E_SHAPE;
  const long long blocks = ((long long)n + 127) / 128 * d->batch * d->heads;
  if (blocks > 0x7FFFFFFFLL) return RQ_E_SHAPE;
  // 32-bit byte offsets of the range-checked loads: one (b, h) of K, V and V^T
  if ((unsigned long long)(n + 64) * d->head_dim * 2 > 0x7FFFFFFFull) return RQ_E_SHAPE;
  if (!ws || ws_bytes < prefill_workspace_bytes(d->batch, d->heads, d->head_dim, n) || ((uintptr_t)ws & 255) != 0)
    return RQ_E_WORKSPACE;
  PrefillParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.lens = lens;
  p.out = out;
  p.vt = static_cast<uint16_t*>(ws);
  p.dev_err = dev_err;
  p.scale_log2 = softmax_scale * kLog2e;
  p.B = d->batch;
  p.H = d->heads;
  p.T = n;
  p.Tp = (n + 63) / 64 * 64;
  return launch_prefill(p, d->head_dim, stream) == 0 ? RQ_OK : RQ_E_HIP;
}

}  // extern "C"
