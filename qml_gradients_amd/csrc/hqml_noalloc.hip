// Allocation-free training step for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// hqml_train_step_noalloc runs the whole-circuit training step (n <= 13: the circuit of
// one sample per workgroup) with the same kernels, in the same order, as
// hqml_train_step on a context: table preparation, the whole-circuit kernel (forward,
// <O>, adjoint statistics), then <O>, the loss and the gradient reduced in one launch.  What a
// context keeps in its workspace (tables, per-sample statistics, sums) lives here in one
// fixed device buffer, `scratch`, of HQML_NOALLOC_SCRATCH_BYTES.  Each GPU holds its own
// copy from the moment the library's code is loaded on it until the process ends; the
// entry point allocates nothing.  Every call on a GPU shares that GPU's copy and leaves
// its contents behind; every part is written before it is read within a call, so
// nothing needs clearing, and calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/hqml.h"
#include "hqml_host.hpp"

// One copy per GPU; host code reaches it only through the address hipGetSymbolAddress
// returns on that GPU (g_scratch below).
static __device__ __align__(256) unsigned char scratch[HQML_NOALLOC_SCRATCH_BYTES];

namespace hqml {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_setup_mu;
// Device address of `scratch` on each GPU, from hipGetSymbolAddress with that GPU
// current (nullptr: not set up yet).  Host code uses these, never the array's name.
char *g_scratch[kMaxDevices];

// Once per device, with the device current: look up this GPU's copy of the scratch
// buffer and allow the whole-circuit kernel its dynamic LDS.
int setup_device(int dev, char **out, std::string *err)
{
    std::lock_guard<std::mutex> lock(g_setup_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
            return HQML_ERR_HIP;
        }
        e = configure_small();
        if (e != hipSuccess) {
            *err = std::string("whole-circuit kernel set-up: ") + hipGetErrorString(e);
            return HQML_ERR_HIP;
        }
        g_scratch[dev] = static_cast<char *>(p);
    }
    *out = g_scratch[dev];
    return HQML_OK;
}

// Consecutive 256-byte-aligned parts of the scratch buffer.
struct Carve {
    char *base;
    size_t used = 0;
    void *take(size_t bytes)
    {
        void *p = base ? base + used : nullptr;
        used += (bytes + 255) & ~(size_t)255;
        return p;
    }
};

struct Parts {
    double *zyz;
    unsigned char *frame;
    void *rot_tf, *dw;
    double *H;
    void *init_u, *e_part;
    double *S, *dlde;
};

// The parts a step of B samples needs (base == nullptr: sizes only); returns the bytes.
size_t carve_parts(char *base, int B, int L, int n, size_t rb, Parts *p)
{
    Carve c{base};
    const size_t Ln = (size_t)L * n, b = (size_t)B;
    p->zyz = static_cast<double *>(c.take(Ln * 6 * 8));
    p->frame = static_cast<unsigned char *>(c.take(Ln));
    p->rot_tf = c.take(Ln * 2 * rb);
    p->dw = c.take(Ln * 4 * rb);
    p->H = static_cast<double *>(c.take(Ln * 9 * 8));
    p->init_u = c.take(b * n * 4 * rb);
    p->e_part = c.take(b * rb);
    p->S = static_cast<double *>(c.take(b * Ln * 3 * 8));
    p->dlde = static_cast<double *>(c.take(b * 8));
    return c.used;
}

int noalloc_fail(int code, const std::string &msg)
{
    set_thread_error(msg);
    return code;
}

}  // namespace
}  // namespace hqml

using namespace hqml;

extern "C" int hqml_train_step_noalloc(const hqml_config *cfg, int B, const float *x, const float *theta,
                                       const float *y, float *expz, float *loss, float *grad)
{
    set_thread_error("");
    Plan plan;
    std::string err;
    int rc = validate_config(cfg, &plan, &err);
    if (rc != HQML_OK) return noalloc_fail(rc, err);
    if (!plan.small || cfg->fusion != HQML_FUSED)
        return noalloc_fail(HQML_ERR_UNSUPPORTED, "hqml_train_step_noalloc covers the fused whole-circuit sizes "
                                                  "only (n_qubits <= 13)");
    if (B < 1 || B > cfg->max_batch) return noalloc_fail(HQML_ERR_ARG, "B must be in 1..max_batch");
    if (cfg->device < 0 || cfg->device >= kMaxDevices) return noalloc_fail(HQML_ERR_ARG, "device ordinal out of range");
    const int n = plan.n, L = plan.L, r64 = cfg->compute == HQML_COMPUTE_FP64 ? 1 : 0;
    const size_t rb = r64 ? 8 : 4;
    Parts parts;
    const size_t need = carve_parts(nullptr, B, L, n, rb, &parts);
    if (need > (size_t)HQML_NOALLOC_SCRATCH_BYTES)
        return noalloc_fail(HQML_ERR_ARG, "batch " + std::to_string(B) + " of a " + std::to_string(n) + "-qubit, " +
                                              std::to_string(L) + "-layer circuit needs " + std::to_string(need) +
                                              " scratch bytes, more than HQML_NOALLOC_SCRATCH_BYTES (" +
                                              std::to_string((size_t)HQML_NOALLOC_SCRATCH_BYTES) + ")");
    hipError_t e = hipSetDevice(cfg->device);
    if (e != hipSuccess) return noalloc_fail(HQML_ERR_HIP, std::string("hipSetDevice: ") + hipGetErrorString(e));
    const size_t nq = (size_t)n, np = (size_t)L * nq * 3 * sizeof(float);
    if ((rc = check_device_array(cfg->device, x, (size_t)B * nq * sizeof(float), "x", &err)) ||
        (rc = check_device_array(cfg->device, theta, np, "theta", &err)) ||
        (rc = check_device_array(cfg->device, y, (size_t)B * sizeof(float), "y", &err)) ||
        (rc = check_device_array(cfg->device, expz, (size_t)B * sizeof(float), "expz", &err)) ||
        (rc = check_device_array(cfg->device, loss, sizeof(float), "loss", &err)) ||
        (rc = check_device_array(cfg->device, grad, np, "grad", &err)))
        return noalloc_fail(rc, err);
    char *base = nullptr;
    if ((rc = setup_device(cfg->device, &base, &err))) return noalloc_fail(rc, err);
    carve_parts(base, B, L, n, rb, &parts);

    hipStream_t st = reinterpret_cast<hipStream_t>(cfg->stream);
    const int ent = cfg->entangler == HQML_ENT_CNOT ? 1 : 0;
    e = launch_prep(theta, x, 0, L, n, B, parts.zyz, parts.frame, parts.rot_tf, parts.dw, parts.H, parts.init_u, ent,
                    r64, st);
    if (e != hipSuccess) return noalloc_fail(HQML_ERR_HIP, std::string("table preparation: ") + hipGetErrorString(e));
    SmallArgs a{};
    a.init_u = parts.init_u;
    a.rot_tf = parts.rot_tf;
    a.dw = parts.dw;
    a.psi_save = nullptr;   // read or written only by forward-only / backward-only launches
    a.e_out = parts.e_part;
    a.stats = parts.S;
    a.n = n;
    a.L = L;
    a.mode = 2;
    a.ent = ent;
    bool neg = false;
    config_observable(cfg, plan, &a.obs, &a.obs_x, &neg);
    e = launch_small(a, B, r64, st);
    if (e != hipSuccess) return noalloc_fail(HQML_ERR_HIP, std::string("small-circuit kernel: ") + hipGetErrorString(e));
    e = launch_small_reduce(parts.e_part, r64, B, y, expz, loss, 0, parts.dlde, parts.S, parts.H, L, n, grad, st);
    if (e != hipSuccess)
        return noalloc_fail(HQML_ERR_HIP, std::string("E and gradient reduction: ") + hipGetErrorString(e));
    return HQML_OK;
}
