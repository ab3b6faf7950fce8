// ddh_internal.h - plan state and device descriptors shared by the library's
// translation units (map builder, exchange kernels, C ABI). Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/ddh.h"

namespace ddh {

// Work-group size of every exchange kernel: four 64-wide wavefronts.
constexpr int kBlock = 256;

// Control words, each on its own 256-byte line (index in uint32 units).
enum CtrlWord : int {
    kCtrlEpoch = 0,    // last completed pass number
    kCtrlTicket = 64,  // next work ticket of the running launch
    kCtrlDone = 128,   // work-groups that left the running launch
    kCtrlXDone = 192,  // coordinate items completed in a fused step launch
    kCtrlError = 256,  // first device-side error code (0 = none)
    kCtrlWords = 320
};

// One (sender S, pulse p) map: 64 bytes, read with scalar loads.
struct DItem {
    int32_t src_base;  // first slot of sender S
    int32_t dst_base;  // first slot of the region at receiver R
    int32_t map_off;   // first entry of the map in the map array
    int32_t send;      // map entries
    int32_t comp;      // pulse dimension d
    int32_t do_shift;  // 1: component d gets + shift
    float shift;       // L_d
    int32_t S, R, p;
    int32_t nchunks;   // chunks of this item (same in every chunk table)
    int32_t pad[5];
};
static_assert(sizeof(DItem) == 64, "DItem layout");

// One work chunk: a contiguous entry range of one item's map. 32 bytes.
struct DChunk {
    int32_t item;
    int32_t begin, end;  // entry range [begin, end) of the item's map
    uint32_t wait_a;     // coords: pulses q whose region at S must be complete
                         // forces: later pulses q whose (S, q) item must be done
    uint32_t wait_b;     // forces: later pulses q whose (R, q) item must be done
    int32_t pad[3];
};
static_assert(sizeof(DChunk) == 32, "DChunk layout");

// Kernel arguments of one exchange launch (passed by value).
struct XArgs {
    float* x;
    float* f;
    const int32_t* maps;
    const DItem* items;
    const DChunk* xchunks;
    const DChunk* fchunks;
    int32_t x_begin, x_end;  // ticket range of coordinate chunks
    int32_t f_begin, f_end;  // ticket range of force chunks
    uint32_t* ctrl;
    uint32_t* xflag;  // [R * P + p] = pass number once region p of R is filled
    uint32_t* fflag;  // [S * P + p] = pass number once item (S, p) has added
    uint32_t* xcnt;   // per-item chunk completion counters (self-resetting)
    uint32_t* fcnt;
    int32_t P;
    int32_t n_items;
    int32_t bump_epoch;     // this launch ends the pass: publish its number
    int32_t force_timeout;  // waits target a value nobody writes
    uint32_t spin_limit;
};

struct Geometry {
    int n[3] = {1, 1, 1};
    float L[3] = {0, 0, 0};
    float rc = 0, cell = 0, inv_c = 0;
    std::vector<float> b[3];      // boundaries, n[d] + 1 per dimension
    std::vector<int> ncell[3];    // sort cells across domain index i of d
    int ndom = 1;
    int P = 0;
    int pdim[DDH_MAX_PULSES] = {0};
    int pk[DDH_MAX_PULSES] = {0};
    void coords(int D, int c[3]) const {
        c[0] = D % n[0];
        c[1] = (D / n[0]) % n[1];
        c[2] = D / (n[0] * n[1]);
    }
    int index(const int c[3]) const { return c[0] + n[0] * (c[1] + n[1] * c[2]); }
};

// A device allocation owned by the plan.
struct DevBuf {
    void* p = nullptr;
    size_t bytes = 0;
};

struct Plan {
    int device = 0;
    int n_cu = 256;
    Geometry g;
    bool built = false;
    int32_t n_atoms = 0;
    int64_t n_slots = 0;
    int64_t n_halo = 0;
    int32_t mode = DDH_MODE_FUSED;

    // tuning
    int chunk_req = 0;
    int grid_req = 0;
    uint32_t spin_limit = 1u << 20;
    int force_timeout = 0;
    int refined_waits = 1;
    int chunk = 256;  // entries per chunk in use

    // host copies of the layout
    std::vector<int64_t> base;     // per domain
    std::vector<int32_t> nhome, ntotal;
    std::vector<int32_t> send, split, recv, roff, shift;  // [S * P + p]
    std::vector<int64_t> map_off;  // [S * P + p]
    std::vector<DItem> items;      // [S * P + p]
    std::vector<DChunk> xch_fused, xch_pulse, fch;
    std::vector<int32_t> xpulse_begin, fpulse_begin;  // per pulse ranges (+1)

    // device state
    int32_t* d_maps = nullptr;     // all maps, pulse-major
    int32_t* d_slot_gid = nullptr; // global id per slot
    int32_t* d_home_gid = nullptr; // home atoms in slot order, all domains
    int32_t* d_home_slot = nullptr;
    DItem* d_items = nullptr;
    DChunk* d_xch_fused = nullptr;
    DChunk* d_xch_pulse = nullptr;
    DChunk* d_fch = nullptr;
    uint32_t* d_ctrl = nullptr;    // control words + flags + counters
    uint32_t* d_xflag = nullptr;
    uint32_t* d_fflag = nullptr;
    uint32_t* d_xcnt = nullptr;
    uint32_t* d_fcnt = nullptr;
    std::vector<void*> owned;      // every hipMalloc of the built state

    // graph replay cache: (op, x, f, mode) -> executable graph
    hipStream_t capture_stream = nullptr;
    std::map<std::tuple<int, void*, void*, int>, hipGraphExec_t> graphs;
};

// error reporting (thread-local text)
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);

#define DDH_HIP(call)                                     \
    do {                                                  \
        hipError_t _e = (call);                           \
        if (_e != hipSuccess) return ddh::hip_fail(_e, #call); \
    } while (0)

// map builder (ddh_build.hip)
int build_maps(Plan* plan, const float* xg, int32_t n_atoms, hipStream_t stream);
void free_built(Plan* plan);

// exchange launches (ddh_exchange.hip)
enum Op : int { kOpCoords = 1, kOpForces = 2, kOpStep = 3 };
int enqueue_exchange(Plan* plan, int op, float* x, float* f, hipStream_t stream);
int enqueue_gather_home(Plan* plan, const float* xg, float* x, hipStream_t stream);

}  // namespace ddh
