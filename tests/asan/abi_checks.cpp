// abi_checks.cpp -- drives every argument check of the C ABI on the host.
//
// Built together with vc_api.hip and launch_stubs.cpp under the host
// AddressSanitizer and UndefinedBehaviorSanitizer.  Each case calls one entry
// point with one bad argument (or with all arguments valid) and checks the
// status and the message vc_last_error gives.  No pointer handed over here
// is dereferenced by the library: tensors and workspaces are plain host
// buffers, or addresses of the right alignment with a size that is only a
// number.  Calls that pass every check end in the launch stubs (or, with no
// GPU, in the device check) and return VC_ERR_DEVICE.
//
// Prints one line per case and "abi_checks: N cases, F failures"; the exit
// status is the number of failures (0 when all hold).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <string>
#include <thread>
#include <vector>

#include "vc.h"

namespace {

int g_cases = 0;
int g_fail = 0;

void expect(const char* name, vc_status got, vc_status want, const char* msg_part) {
  ++g_cases;
  const std::string msg = vc_last_error();
  bool good = got == want;
  if (good && msg_part) good = msg.find(msg_part) != std::string::npos;
  if (good && want == VC_OK) good = msg.empty();
  if (!good) ++g_fail;
  std::printf("%s %-48s %-18s %s\n", good ? "ok  " : "FAIL", name, vc_status_string(got), msg.c_str());
}

// A contiguous [B,S,H,128] descriptor.
vc_desc desc(int B, int S, int H, int dtype = VC_BF16) {
  vc_desc d;
  std::memset(&d, 0, sizeof d);
  d.B = B;
  d.S = S;
  d.H = H;
  d.D = 128;
  d.dtype = dtype;
  d.sH = 128;
  d.sS = static_cast<int64_t>(H) * 128;
  d.sB = static_cast<int64_t>(S) * H * 128;
  return d;
}

vc_v_opts opts(int k = 8, int iters = 3, float beta = 0.0f, int smooth = 1, int fmt = VC_V_E4M3) {
  vc_v_opts o;
  std::memset(&o, 0, sizeof o);
  o.smooth = smooth;
  o.k = k;
  o.iters = iters;
  o.v_format = fmt;
  o.seed = 7;
  o.repair_budget = beta;
  return o;
}

// An address with the given alignment that is never dereferenced.
const void* fake_ptr(uintptr_t align) { return reinterpret_cast<const void*>(uintptr_t{1} << 40 | align); }

void layout_cases() {
  vc_ws_layout L;
  vc_desc d = desc(1, 1000, 2);
  vc_v_opts o = opts();
  expect("layout: out NULL", vc_workspace_layout(&d, &o, nullptr), VC_ERR_ARG, "layout output");
  expect("layout: desc NULL", vc_workspace_layout(nullptr, &o, &L), VC_ERR_ARG, "descriptor is NULL");
  expect("layout: opts NULL", vc_workspace_layout(&d, nullptr, &L), VC_ERR_ARG, "options pointer");

  struct DescCase {
    const char* name;
    std::function<void(vc_desc&)> edit;
    vc_status want;
    const char* part;
  };
  const std::vector<DescCase> dcases = {
      {"desc: B = 0", [](vc_desc& x) { x.B = 0; }, VC_ERR_ARG, "must be >= 1"},
      {"desc: S = 0", [](vc_desc& x) { x.S = 0; }, VC_ERR_ARG, "must be >= 1"},
      {"desc: H = -1", [](vc_desc& x) { x.H = -1; }, VC_ERR_ARG, "must be >= 1"},
      {"desc: D = 64", [](vc_desc& x) { x.D = 64; }, VC_ERR_UNSUPPORTED, "head dimension"},
      {"desc: dtype = 7", [](vc_desc& x) { x.dtype = 7; }, VC_ERR_UNSUPPORTED, "dtype"},
      {"desc: S = 2^24 + 1", [](vc_desc& x) { x.S = (1 << 24) + 1; }, VC_ERR_UNSUPPORTED, "exceeds"},
      {"desc: B*H = 2^21", [](vc_desc& x) { x.B = 2048; x.H = 1024; }, VC_ERR_UNSUPPORTED, "B*H"},
      {"desc: H = 65536", [](vc_desc& x) { x.H = 65536; }, VC_ERR_UNSUPPORTED, "each be <="},
      {"desc: B = 65536", [](vc_desc& x) { x.B = 65536; }, VC_ERR_UNSUPPORTED, "each be <="},
      {"desc: sS < 0", [](vc_desc& x) { x.sS = -256; }, VC_ERR_ARG, "negative stride"},
      {"desc: sB odd", [](vc_desc& x) { x.sB += 1; }, VC_ERR_ARG, "multiples of 8"},
      {"desc: sH = 4", [](vc_desc& x) { x.sH = 4; }, VC_ERR_ARG, "multiples of 8"},
  };
  for (const DescCase& c : dcases) {
    vc_desc x = desc(1, 1000, 2);
    c.edit(x);
    expect(c.name, vc_workspace_layout(&x, &o, &L), c.want, c.part);
  }

  struct OptCase {
    const char* name;
    vc_v_opts o;
    vc_status want;
    const char* part;
  };
  const std::vector<OptCase> ocases = {
      {"opts: smooth = 2", opts(8, 3, 0.0f, 2), VC_ERR_ARG, "smooth"},
      {"opts: k = 0", opts(0), VC_ERR_ARG, "1 <= k <= S"},
      {"opts: k > S", opts(1001), VC_ERR_ARG, "1 <= k <= S"},
      {"opts: k = 65", opts(65), VC_ERR_UNSUPPORTED, "clusters"},
      {"opts: iters = -1", opts(8, -1), VC_ERR_ARG, "iters"},
      {"opts: iters = 65", opts(8, 65), VC_ERR_ARG, "iters"},
      {"opts: beta = -0.1", opts(8, 3, -0.1f), VC_ERR_ARG, "repair_budget"},
      {"opts: beta = 1", opts(8, 3, 1.0f), VC_ERR_ARG, "repair_budget"},
      {"opts: beta = NaN", opts(8, 3, std::nanf("")), VC_ERR_ARG, "repair_budget"},
      {"opts: v_format = 2", opts(8, 3, 0.0f, 1, 2), VC_ERR_ARG, "v_format"},
      {"opts: MXFP4 with repair", opts(8, 3, 0.01f, 1, VC_V_MXFP4), VC_ERR_UNSUPPORTED, "no repair"},
  };
  for (const OptCase& c : ocases) expect(c.name, vc_workspace_layout(&d, &c.o, &L), c.want, c.part);

  // k, iters are not read without smoothing
  const vc_v_opts plain = opts(0, -5, 0.0f, 0);
  expect("opts: smooth = 0 ignores k and iters", vc_workspace_layout(&d, &plain, &L), VC_OK, nullptr);

  // A valid layout: 256-byte aligned regions in order, sizes of the stated
  // element counts, for shapes from one token up to the largest supported.
  struct Shape {
    int B, S, H, k;
    float beta;
  };
  const Shape shapes[] = {{1, 1, 1, 1, 0.0f},      {1, 127, 1, 5, 0.5f},     {2, 4096, 8, 32, 0.005f},
                          {1, 73397, 56, 32, 0.0f}, {1, 1 << 24, 64, 64, 0.01f}, {1024, 129, 1024, 64, 0.0f}};
  for (const Shape& s : shapes) {
    vc_desc x = desc(s.B, s.S, s.H);
    vc_v_opts ox = opts(s.k, 5, s.beta);
    char name[96];
    std::snprintf(name, sizeof name, "layout: B=%d S=%d H=%d k=%d beta=%g", s.B, s.S, s.H, s.k, s.beta);
    const vc_status st = vc_workspace_layout(&x, &ox, &L);
    expect(name, st, VC_OK, nullptr);
    if (st != VC_OK) continue;
    const size_t off[] = {L.q8,     L.q_scale, L.k8,     L.k_scale, L.v8,     L.v_mean, L.v_muop,    L.hdr,
                          L.assign, L.perm,    L.rep_pos, L.rep_k8, L.rep_ks, L.rep_e8, L.attn_part, L.scratch};
    const int nblk = (s.S + 127) / 128;
    const int nrep = s.beta > 0 ? std::min<int>(s.S, static_cast<int>(std::ceil(static_cast<double>(s.beta) * s.S))) : 0;
    const size_t BH = static_cast<size_t>(s.B) * s.H;
    bool good = L.nblk == nblk && L.nrep == nrep && L.nrep_pad == 128 * ((nrep + 127) / 128) && L.q8 == 0;
    for (size_t i = 0; i < sizeof off / sizeof off[0]; ++i) {
      good = good && off[i] % 256 == 0 && off[i] <= L.total;
      if (i) good = good && off[i] >= off[i - 1];
    }
    good = good && L.q_scale - L.q8 >= BH * nblk * 16384 && L.k8 - L.q_scale >= BH * nblk * 4;
    good = good && L.perm - L.assign >= BH * s.S * 4 && L.rep_pos - L.perm >= BH * s.S * 4;
    good = good && L.rep_k8 - L.rep_pos >= BH * L.nrep_pad * 4 && L.total > L.scratch;
    ++g_cases;
    if (!good) ++g_fail;
    std::printf("%s %-48s total %zu bytes\n", good ? "ok  " : "FAIL", "  regions aligned and sized", L.total);
  }
}

void entry_cases() {
  // buffers the library sees but never reads on the host
  const int B = 1, S = 1000, H = 2;
  vc_desc d = desc(B, S, H);
  vc_v_opts o = opts();
  vc_ws_layout L;
  if (vc_workspace_layout(&d, &o, &L) != VC_OK) {
    ++g_fail;
    return;
  }
  std::vector<uint16_t> v(static_cast<size_t>(B) * S * H * 128 + 8);
  uint16_t* vp = reinterpret_cast<uint16_t*>((reinterpret_cast<uintptr_t>(v.data()) + 15) & ~uintptr_t{15});
  void* ws = std::aligned_alloc(256, (L.total + 255) / 256 * 256);
  uint8_t* wsb = static_cast<uint8_t*>(ws);

  expect("prepare_v: desc NULL", vc_prepare_v(nullptr, vp, &o, ws, L.total, nullptr), VC_ERR_ARG, "descriptor");
  expect("prepare_v: opts NULL", vc_prepare_v(&d, vp, nullptr, ws, L.total, nullptr), VC_ERR_ARG, "options");
  expect("prepare_v: v NULL", vc_prepare_v(&d, nullptr, &o, ws, L.total, nullptr), VC_ERR_ARG, "v is NULL");
  expect("prepare_v: v misaligned", vc_prepare_v(&d, vp + 1, &o, ws, L.total, nullptr), VC_ERR_ARG, "16-byte");
  expect("prepare_v: ws NULL", vc_prepare_v(&d, vp, &o, nullptr, L.total, nullptr), VC_ERR_ARG, "workspace is NULL");
  expect("prepare_v: ws misaligned", vc_prepare_v(&d, vp, &o, wsb + 16, L.total, nullptr), VC_ERR_ARG, "256-byte");
  expect("prepare_v: ws one byte short", vc_prepare_v(&d, vp, &o, ws, L.total - 1, nullptr), VC_ERR_WORKSPACE,
         "needs");
  expect("prepare_v: valid", vc_prepare_v(&d, vp, &o, ws, L.total, nullptr), VC_ERR_DEVICE, nullptr);

  expect("noalloc: v NULL", vc_prepare_v_noalloc(&d, nullptr, &o, ws, L.scratch, nullptr), VC_ERR_ARG, "v is NULL");
  expect("noalloc: ws short of the scratch offset", vc_prepare_v_noalloc(&d, vp, &o, ws, L.scratch - 1, nullptr),
         VC_ERR_WORKSPACE, "needs");
  expect("noalloc: valid", vc_prepare_v_noalloc(&d, vp, &o, ws, L.scratch, nullptr), VC_ERR_DEVICE, nullptr);
  {
    // a shape whose scratch exceeds the static array (checked before the device)
    vc_desc big = desc(1, 1 << 22, 64);
    vc_v_opts ob = opts(64, 3);
    vc_ws_layout Lb;
    const vc_status st = vc_workspace_layout(&big, &ob, &Lb);
    expect("noalloc: big shape layout", st, VC_OK, nullptr);
    if (st == VC_OK && Lb.total - Lb.scratch > VC_NOALLOC_SCRATCH_BYTES)
      expect("noalloc: scratch above the static array",
             vc_prepare_v_noalloc(&big, fake_ptr(16), &ob, const_cast<void*>(fake_ptr(256)), Lb.scratch, nullptr),
             VC_ERR_UNSUPPORTED, "static array");
    else
      expect("noalloc: big shape needs more scratch than the array", VC_ERR_ARG, VC_OK, nullptr);
  }

  vc_desc dk = d;
  vc_desc dbad = desc(B, S + 1, H);
  expect("prepare_qk: q desc NULL", vc_prepare_qk(nullptr, vp, &dk, vp, &o, ws, L.scratch, nullptr), VC_ERR_ARG,
         "q: descriptor");
  expect("prepare_qk: k desc NULL", vc_prepare_qk(&d, vp, nullptr, vp, &o, ws, L.scratch, nullptr), VC_ERR_ARG,
         "k: descriptor");
  expect("prepare_qk: shapes differ", vc_prepare_qk(&d, vp, &dbad, vp, &o, ws, L.scratch, nullptr), VC_ERR_ARG,
         "same B, S, H");
  {
    vc_desc dq = d;
    dq.dtype = VC_F16;  // q and k may differ in dtype and strides
    dq.sS = 2 * d.sS;
    dq.sB = 2 * d.sB;
    expect("prepare_qk: q f16, k bf16, q strided", vc_prepare_qk(&dq, vp, &dk, vp, &o, ws, L.scratch, nullptr),
           VC_ERR_DEVICE, nullptr);
  }
  expect("prepare_qk: q NULL", vc_prepare_qk(&d, nullptr, &dk, vp, &o, ws, L.scratch, nullptr), VC_ERR_ARG,
         "q is NULL");
  expect("prepare_qk: k misaligned", vc_prepare_qk(&d, vp, &dk, vp + 4, &o, ws, L.scratch, nullptr), VC_ERR_ARG,
         "k must be 16-byte");
  expect("prepare_qk: ws short", vc_prepare_qk(&d, vp, &dk, vp, &o, ws, L.scratch - 256, nullptr), VC_ERR_WORKSPACE,
         "needs");
  expect("prepare_qk: valid", vc_prepare_qk(&d, vp, &dk, vp, &o, ws, L.scratch, nullptr), VC_ERR_DEVICE, nullptr);

  vc_attn_opts ao{0.0f, 0};
  vc_desc dof = desc(B, S, H, VC_F16);
  expect("attention: out desc NULL", vc_attention_fwd(nullptr, vp, &o, &ao, ws, L.scratch, nullptr), VC_ERR_ARG,
         "out: descriptor");
  expect("attention: out f16", vc_attention_fwd(&dof, vp, &o, &ao, ws, L.scratch, nullptr), VC_ERR_UNSUPPORTED,
         "out: dtype");
  expect("attention: opts NULL", vc_attention_fwd(&d, vp, nullptr, &ao, ws, L.scratch, nullptr), VC_ERR_ARG,
         "options");
  expect("attention: out NULL", vc_attention_fwd(&d, nullptr, &o, &ao, ws, L.scratch, nullptr), VC_ERR_ARG,
         "out is NULL");
  expect("attention: ws NULL", vc_attention_fwd(&d, vp, &o, &ao, nullptr, L.scratch, nullptr), VC_ERR_ARG,
         "workspace is NULL");
  expect("attention: ws short", vc_attention_fwd(&d, vp, &o, &ao, ws, L.scratch - 1, nullptr), VC_ERR_WORKSPACE,
         "needs");
  const float bad_sm[] = {-1.0f, std::nanf(""), INFINITY};
  for (float sm : bad_sm) {
    vc_attn_opts b{sm, 0};
    char name[64];
    std::snprintf(name, sizeof name, "attention: sm_scale = %g", sm);
    expect(name, vc_attention_fwd(&d, vp, &o, &b, ws, L.scratch, nullptr), VC_ERR_ARG, "sm_scale");
  }
  expect("attention: aopts NULL (default scale)", vc_attention_fwd(&d, vp, &o, nullptr, ws, L.scratch, nullptr),
         VC_ERR_DEVICE, nullptr);
  expect("attention: valid", vc_attention_fwd(&d, vp, &o, &ao, ws, L.scratch, nullptr), VC_ERR_DEVICE, nullptr);
  {
    // more attention workgroups than one launch holds (checked before the device)
    vc_desc huge = desc(16, 4096, 65535);
    vc_v_opts oh = opts(8, 1, 0.0f, 0);
    vc_ws_layout Lh;
    const vc_status st = vc_workspace_layout(&huge, &oh, &Lh);
    expect("attention: huge shape layout", st, VC_OK, nullptr);
    if (st == VC_OK)
      expect("attention: too many workgroups",
             vc_attention_fwd(&huge, const_cast<void*>(fake_ptr(16)), &oh, &ao, fake_ptr(256), Lh.scratch, nullptr),
             VC_ERR_UNSUPPORTED, "attention workgroups");
  }
  std::free(ws);
}

void misc_cases() {
  const vc_status all[] = {VC_OK, VC_ERR_ARG, VC_ERR_UNSUPPORTED, VC_ERR_WORKSPACE, VC_ERR_DEVICE};
  const char* names[] = {"VC_OK", "VC_ERR_ARG", "VC_ERR_UNSUPPORTED", "VC_ERR_WORKSPACE", "VC_ERR_DEVICE"};
  for (int i = 0; i < 5; ++i) {
    ++g_cases;
    const bool good = std::strcmp(vc_status_string(all[i]), names[i]) == 0;
    if (!good) ++g_fail;
    std::printf("%s status string %-34s %s\n", good ? "ok  " : "FAIL", names[i], vc_status_string(all[i]));
  }
  ++g_cases;
  if (std::strcmp(vc_status_string(static_cast<vc_status>(99)), "VC_ERR_UNKNOWN") != 0) ++g_fail;
  ++g_cases;
  if (!vc_version() || !*vc_version()) ++g_fail;
  std::printf("ok   version %s\n", vc_version());

  // the last error is per thread, and a successful call clears it
  vc_ws_layout L;
  vc_desc d = desc(1, 10, 1);
  vc_v_opts o = opts(4, 1);
  vc_workspace_layout(nullptr, &o, &L);
  std::string other = "unset";
  std::thread t([&]() { other = vc_last_error(); });
  t.join();
  ++g_cases;
  const bool per_thread = other.empty() && std::strstr(vc_last_error(), "descriptor is NULL");
  if (!per_thread) ++g_fail;
  std::printf("%s last error is per thread\n", per_thread ? "ok  " : "FAIL");
  expect("a valid call clears the last error", vc_workspace_layout(&d, &o, &L), VC_OK, nullptr);
}

}  // namespace

int main() {
  layout_cases();
  entry_cases();
  misc_cases();
  std::printf("abi_checks: %d cases, %d failures\n", g_cases, g_fail);
  return g_fail;
}
