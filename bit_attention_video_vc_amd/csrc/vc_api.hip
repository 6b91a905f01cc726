// vc_api.hip -- the C ABI of libvc.so: argument validation, workspace layout
// and launch sequencing.  Every check here runs before any HIP call, so an
// invalid call returns a status without touching the device.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "vc_common.hpp"
#include "vc_kernels.hpp"

namespace {

thread_local std::string g_last_error;

vc_status fail(vc_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

vc_status ok() {
  g_last_error.clear();
  return VC_OK;
}

constexpr int64_t kMaxS = 1 << 24;
constexpr int64_t kMaxBH = 1 << 20;
constexpr int kMaxGridYZ = 65535;

vc_status check_desc(const vc_desc* d, const char* name) {
  if (!d) return fail(VC_ERR_ARG, "%s: descriptor is NULL", name);
  if (d->B < 1 || d->S < 1 || d->H < 1) return fail(VC_ERR_ARG, "%s: B, S, H must be >= 1 (got %d, %d, %d)", name, d->B, d->S, d->H);
  if (d->D != vc::kD) return fail(VC_ERR_UNSUPPORTED, "%s: head dimension must be 128 (got %d)", name, d->D);
  if (d->dtype != VC_F16 && d->dtype != VC_BF16) return fail(VC_ERR_UNSUPPORTED, "%s: dtype must be VC_F16 or VC_BF16", name);
  if (d->S > kMaxS) return fail(VC_ERR_UNSUPPORTED, "%s: S = %d exceeds %lld", name, d->S, (long long)kMaxS);
  if (static_cast<int64_t>(d->B) * d->H > kMaxBH) return fail(VC_ERR_UNSUPPORTED, "%s: B*H exceeds %lld", name, (long long)kMaxBH);
  // heads and batches index the second and third grid dimensions (<= 65535 each)
  if (d->H > kMaxGridYZ || d->B > kMaxGridYZ)
    return fail(VC_ERR_UNSUPPORTED, "%s: B and H must each be <= %d", name, kMaxGridYZ);
  if (d->sB < 0 || d->sS < 0 || d->sH < 0) return fail(VC_ERR_ARG, "%s: negative stride", name);
  if ((d->sB % 8) || (d->sS % 8) || (d->sH % 8)) return fail(VC_ERR_ARG, "%s: strides must be multiples of 8 elements (16 bytes)", name);
  return VC_OK;
}

struct Plan {
  int B, S, H, k, nblk, nrep, nrep_pad;
  vc::AttnSplit split;
  vc_ws_layout lay;
  vc::Scratch scr;
};

vc_status check_opts(const vc_v_opts* o, int S) {
  if (!o) return fail(VC_ERR_ARG, "options pointer is NULL");
  if (o->smooth != 0 && o->smooth != 1) return fail(VC_ERR_ARG, "smooth must be 0 or 1");
  if (o->smooth) {
    if (o->k < 1 || o->k > S) return fail(VC_ERR_ARG, "k must satisfy 1 <= k <= S (k=%d, S=%d)", o->k, S);
    if (o->k > vc::kMaxK) return fail(VC_ERR_UNSUPPORTED, "k > %d clusters is not supported", vc::kMaxK);
    if (o->iters < 0 || o->iters > 64) return fail(VC_ERR_ARG, "iters must be in [0, 64]");
  }
  if (!(o->repair_budget >= 0.0f && o->repair_budget < 1.0f)) return fail(VC_ERR_ARG, "repair_budget must be in [0, 1)");
  if (o->v_format != VC_V_E4M3 && o->v_format != VC_V_MXFP4) return fail(VC_ERR_ARG, "v_format must be 0 or 1");
  if (o->v_format == VC_V_MXFP4 && o->repair_budget > 0.0f)
    return fail(VC_ERR_UNSUPPORTED, "the MXFP4 residual has no repair");
  return VC_OK;
}

vc_status make_plan(const vc_desc* vd, const vc_v_opts* o, Plan* p) {
  vc_status s = check_desc(vd, "v");
  if (s != VC_OK) return s;
  s = check_opts(o, vd->S);
  if (s != VC_OK) return s;
  p->B = vd->B;
  p->S = vd->S;
  p->H = vd->H;
  p->k = o->smooth ? o->k : 1;
  p->nblk = (vd->S + vc::kBlock - 1) / vc::kBlock;
  p->nrep = 0;
  if (o->repair_budget > 0.0f) {
    const double n = std::ceil(static_cast<double>(o->repair_budget) * vd->S);
    p->nrep = static_cast<int>(n < vd->S ? n : vd->S);
  }
  p->nrep_pad = vc::kBlock * ((p->nrep + vc::kBlock - 1) / vc::kBlock);
  const int64_t BH = static_cast<int64_t>(p->B) * p->H;
  const size_t tiles = static_cast<size_t>(BH) * p->nblk * vc::kTileBytes;
  const size_t per_blk = static_cast<size_t>(BH) * p->nblk;
  vc_ws_layout& L = p->lay;
  std::memset(&L, 0, sizeof L);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = vc::align256(off + bytes);
    return at;
  };
  L.q8 = take(tiles);
  L.q_scale = take(sizeof(float) * per_blk);
  L.k8 = take(tiles);
  L.k_scale = take(sizeof(float) * per_blk);
  L.v8 = take(tiles);
  L.v_mean = take(sizeof(float) * per_blk * vc::kD);
  L.v_muop = take(static_cast<size_t>(BH) * vc::muop_rows(p->nblk) * vc::kMuOpRowBytes);
  L.hdr = take(sizeof(vc_head_hdr) * BH);
  L.assign = take(sizeof(int32_t) * BH * p->S);
  L.perm = take(sizeof(int32_t) * BH * p->S);
  L.rep_pos = take(sizeof(int32_t) * BH * p->nrep_pad);
  L.rep_k8 = take(static_cast<size_t>(BH) * p->nrep_pad * vc::kD);
  L.rep_ks = take(sizeof(float) * BH * p->nrep_pad);
  L.rep_e8 = take(static_cast<size_t>(BH) * p->nrep_pad * vc::kD);
  p->split = vc::attn_split(BH, p->nblk, p->nrep);
  L.attn_part = take(static_cast<size_t>(2) * p->split.tail_wg * vc::kPartBytes);
  p->scr = vc::scratch_layout(BH, p->S, p->k, p->nrep);
  L.scratch = take(p->scr.total);
  L.total = off;
  L.nblk = p->nblk;
  L.nrep = p->nrep;
  L.nrep_pad = p->nrep_pad;
  return VC_OK;
}

// `need`: the bytes a call touches -- the whole layout for vc_prepare_v, the
// regions before the scratch region for every other call.
vc_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(VC_ERR_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(VC_ERR_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(VC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return VC_OK;
}

vc_status check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(VC_ERR_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16) return fail(VC_ERR_ARG, "%s must be 16-byte aligned", name);
  return VC_OK;
}

// Typed pointers into a workspace; the scratch region is at `scr` (the
// workspace's own scratch region unless given).
vc::WsPtrs ws_ptrs(const Plan& p, void* ws, uint8_t* scr = nullptr) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  const vc_ws_layout& L = p.lay;
  if (!scr) scr = base + L.scratch;
  vc::WsPtrs w;
  w.q8 = base + L.q8;
  w.k8 = base + L.k8;
  w.v8 = base + L.v8;
  w.rep_k8 = base + L.rep_k8;
  w.rep_e8 = base + L.rep_e8;
  w.q_scale = reinterpret_cast<float*>(base + L.q_scale);
  w.k_scale = reinterpret_cast<float*>(base + L.k_scale);
  w.v_mean = reinterpret_cast<float*>(base + L.v_mean);
  w.v_muop = base + L.v_muop;
  w.rep_ks = reinterpret_cast<float*>(base + L.rep_ks);
  w.hdr = reinterpret_cast<vc_head_hdr*>(base + L.hdr);
  w.assign = reinterpret_cast<int32_t*>(base + L.assign);
  w.perm = reinterpret_cast<int32_t*>(base + L.perm);
  w.rep_pos = reinterpret_cast<int32_t*>(base + L.rep_pos);
  w.cent = reinterpret_cast<int32_t*>(scr + p.scr.cent);
  w.cent_op = scr + p.scr.cent_op;
  w.cnorm = reinterpret_cast<int32_t*>(scr + p.scr.cnorm);
  w.csum = reinterpret_cast<int64_t*>(scr + p.scr.csum);
  w.ccount = reinterpret_cast<int32_t*>(scr + p.scr.ccount);
  w.chunk_hist = reinterpret_cast<int32_t*>(scr + p.scr.chunk_hist);
  w.chunk_off = reinterpret_cast<int32_t*>(scr + p.scr.chunk_off);
  w.rep_norm = reinterpret_cast<double*>(scr + p.scr.rep_norm);
  w.nblk = p.nblk;
  w.nrep = p.nrep;
  w.nrep_pad = p.nrep_pad;
  return w;
}

vc::TensorArg targ(const vc_desc* d, const void* ptr) {
  vc::TensorArg t;
  t.p = ptr;
  t.sB = d->sB;
  t.sS = d->sS;
  t.sH = d->sH;
  t.dtype = d->dtype;
  return t;
}

// Device check (gfx950 only) and one-time kernel attributes, per device.
constexpr int kMaxDev = 64;
std::once_flag g_dev_once[kMaxDev];
int g_dev_ok[kMaxDev];
std::string g_dev_msg[kMaxDev];

vc_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VC_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDev) return fail(VC_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t prop;
    hipError_t e2 = hipGetDeviceProperties(&prop, dev);
    if (e2 != hipSuccess) {
      g_dev_ok[dev] = 0;
      g_dev_msg[dev] = std::string("hipGetDeviceProperties: ") + hipGetErrorString(e2);
      return;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      g_dev_ok[dev] = 0;
      g_dev_msg[dev] = std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950";
      return;
    }
    g_dev_ok[dev] = 1;
  });
  if (!g_dev_ok[dev]) return fail(g_dev_msg[dev].rfind("device is", 0) == 0 ? VC_ERR_UNSUPPORTED : VC_ERR_DEVICE,
                                  "%s", g_dev_msg[dev].c_str());
  return VC_OK;
}

bool same_shape(const vc_desc* a, const vc_desc* b) { return a->B == b->B && a->S == b->S && a->H == b->H; }

// The scratch of vc_prepare_v_noalloc: a file-scope device array, one copy per
// GPU (each at its own address), held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in):
// the device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and kept per device.
static __device__ __align__(256) uint8_t scratch[VC_NOALLOC_SCRATCH_BYTES];
std::once_flag g_scr_once[kMaxDev];
uint8_t* g_scr_ptr[kMaxDev];
hipError_t g_scr_err[kMaxDev];

// Device address of this device's copy (check_device has validated the
// current device index).
vc_status static_scratch(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VC_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  std::call_once(g_scr_once[dev], [dev]() {
    void* ptr = nullptr;
    g_scr_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scr_ptr[dev] = static_cast<uint8_t*>(ptr);
  });
  if (g_scr_err[dev] != hipSuccess)
    return fail(VC_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(g_scr_err[dev]));
  if (!g_scr_ptr[dev] || reinterpret_cast<uintptr_t>(g_scr_ptr[dev]) % 256)
    return fail(VC_ERR_DEVICE, "static scratch has no 256-byte aligned device address");
  *out = g_scr_ptr[dev];
  return VC_OK;
}

}  // namespace

extern "C" {

#ifndef VC_ABLATION_EXP_CAST
const char* vc_version(void) { return "0.1.0"; }
#else
// the measurement build (FP32 exponential + E4M3 cast instead of ExpCast)
const char* vc_version(void) { return "0.1.0+ablation-exp-cast"; }
#endif

const char* vc_status_string(vc_status s) {
  switch (s) {
    case VC_OK: return "VC_OK";
    case VC_ERR_ARG: return "VC_ERR_ARG";
    case VC_ERR_UNSUPPORTED: return "VC_ERR_UNSUPPORTED";
    case VC_ERR_WORKSPACE: return "VC_ERR_WORKSPACE";
    case VC_ERR_DEVICE: return "VC_ERR_DEVICE";
    default: break;
  }
  return "VC_ERR_UNKNOWN";
}

const char* vc_last_error(void) { return g_last_error.c_str(); }

vc_status vc_workspace_layout(const vc_desc* vd, const vc_v_opts* opts, vc_ws_layout* out) {
  if (!out) return fail(VC_ERR_ARG, "layout output pointer is NULL");
  Plan p;
  vc_status s = make_plan(vd, opts, &p);
  if (s != VC_OK) return s;
  *out = p.lay;
  return ok();
}

vc_status vc_prepare_v(const vc_desc* vd, const void* v, const vc_v_opts* opts, void* ws, size_t ws_bytes,
                       void* stream) {
  Plan p;
  vc_status s = make_plan(vd, opts, &p);
  if (s != VC_OK) return s;
  if ((s = check_ptr(v, "v")) != VC_OK) return s;
  if ((s = check_ws(ws, ws_bytes, p.lay.total)) != VC_OK) return s;
  if ((s = check_device()) != VC_OK) return s;
  const hipError_t e = vc::launch_prepare_v(targ(vd, v), p.B, p.S, p.H, *opts, ws_ptrs(p, ws),
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VC_ERR_DEVICE, "prepare_v launch: %s", hipGetErrorString(e));
  return ok();
}

vc_status vc_prepare_v_noalloc(const vc_desc* vd, const void* v, const vc_v_opts* opts, void* ws, size_t ws_bytes,
                               void* stream) {
  Plan p;
  vc_status s = make_plan(vd, opts, &p);
  if (s != VC_OK) return s;
  if ((s = check_ptr(v, "v")) != VC_OK) return s;
  if ((s = check_ws(ws, ws_bytes, p.lay.scratch)) != VC_OK) return s;
  const size_t need = p.lay.total - p.lay.scratch;
  if (need > VC_NOALLOC_SCRATCH_BYTES)
    return fail(VC_ERR_UNSUPPORTED, "this shape needs %zu bytes of scratch, the static array holds %zu", need,
                static_cast<size_t>(VC_NOALLOC_SCRATCH_BYTES));
  if ((s = check_device()) != VC_OK) return s;
  uint8_t* scr = nullptr;
  if ((s = static_scratch(&scr)) != VC_OK) return s;
  const hipError_t e = vc::launch_prepare_v(targ(vd, v), p.B, p.S, p.H, *opts, ws_ptrs(p, ws, scr),
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VC_ERR_DEVICE, "prepare_v launch: %s", hipGetErrorString(e));
  return ok();
}

vc_status vc_prepare_qk(const vc_desc* qd, const void* q, const vc_desc* kd, const void* k, const vc_v_opts* opts,
                        void* ws, size_t ws_bytes, void* stream) {
  vc_status s = check_desc(qd, "q");
  if (s != VC_OK) return s;
  if ((s = check_desc(kd, "k")) != VC_OK) return s;
  if (!same_shape(qd, kd)) return fail(VC_ERR_ARG, "q and k must have the same B, S, H");
  Plan p;
  if ((s = make_plan(kd, opts, &p)) != VC_OK) return s;
  if ((s = check_ptr(q, "q")) != VC_OK) return s;
  if ((s = check_ptr(k, "k")) != VC_OK) return s;
  if ((s = check_ws(ws, ws_bytes, p.lay.scratch)) != VC_OK) return s;
  if ((s = check_device()) != VC_OK) return s;
  const hipError_t e = vc::launch_prepare_qk(targ(qd, q), targ(kd, k), p.B, p.S, p.H, opts->v_format, ws_ptrs(p, ws),
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VC_ERR_DEVICE, "prepare_qk launch: %s", hipGetErrorString(e));
  return ok();
}

vc_status vc_attention_fwd(const vc_desc* od, void* out, const vc_v_opts* opts, const vc_attn_opts* aopts,
                           const void* ws, size_t ws_bytes, void* stream) {
  vc_status s = check_desc(od, "out");
  if (s != VC_OK) return s;
  if (od->dtype != VC_BF16) return fail(VC_ERR_UNSUPPORTED, "out: dtype must be VC_BF16");
  Plan p;
  if ((s = make_plan(od, opts, &p)) != VC_OK) return s;
  if ((s = check_ptr(out, "out")) != VC_OK) return s;
  if ((s = check_ws(ws, ws_bytes, p.lay.scratch)) != VC_OK) return s;
  float sm = aopts ? aopts->sm_scale : 0.0f;
  if (!(sm >= 0.0f) || std::isinf(sm)) return fail(VC_ERR_ARG, "sm_scale must be finite and >= 0");
  if (sm == 0.0f) sm = static_cast<float>(1.0 / std::sqrt(128.0));
  // whole items, then the tail workgroups; or the short-launch form's query blocks
  const int64_t total = p.split.halves ? static_cast<int64_t>(p.B) * p.H * p.nblk : p.split.whole + p.split.tail_wg;
  if (total > vc::kMaxAttnWorkgroups)
    return fail(VC_ERR_UNSUPPORTED, "B*H*ceil(S/256) = %lld exceeds %lld attention workgroups", (long long)total,
                (long long)vc::kMaxAttnWorkgroups);
  if ((s = check_device()) != VC_OK) return s;
  const vc::WsPtrs w = ws_ptrs(p, const_cast<void*>(ws));
  vc::AttnArgs a;
  a.q8 = w.q8;
  a.q_scale = w.q_scale;
  a.k8 = w.k8;
  a.k_scale = w.k_scale;
  a.v8 = w.v8;
  a.v_muop = w.v_muop;
  a.hdr = w.hdr;
  a.rep_k8 = w.rep_k8;
  a.rep_ks = w.rep_ks;
  a.rep_e8 = w.rep_e8;
  a.out = static_cast<uint16_t*>(out);
  a.osB = od->sB;
  a.osS = od->sS;
  a.osH = od->sH;
  a.S = p.S;
  a.H = p.H;
  a.nblk = p.nblk;
  a.nrep_pad = p.nrep_pad;
  a.whole = static_cast<int>(p.split.whole);
  vc::AttnTail tl;
  tl.tail = p.split.tail;
  tl.tail_wg = p.split.tail_wg;
  tl.per = p.split.per;
  tl.ngrp = p.split.ngrp;
  tl.part = reinterpret_cast<float*>(static_cast<uint8_t*>(const_cast<void*>(ws)) + p.lay.attn_part);
  tl.halves = p.split.halves ? static_cast<int>(total) : 0;
  tl.ka = p.split.ka;
  a.sm_scale = sm;
  a.v_format = opts->v_format;
  const hipError_t e = vc::launch_attention(a, tl, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VC_ERR_DEVICE, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
