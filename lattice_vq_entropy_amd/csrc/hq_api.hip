// hq_api.hip -- host side of libhq: plans, argument checks, kernel launches,
// status, and rate calibration.  See include/hq.h for the contract.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/hq.h"
#include "hq_kernels.h"
#include "hq_ws.h"

struct hq_plan_s {
  int lattice;
  float bps;
  uint64_t seed;
  bool has_alpha;
  float alpha, c_enc, c_dec;
  uint32_t sgn[4];              // bit c: coordinate c of D is -1
  uint32_t sl16[4], sl32[4];    // the same in the kernels' lane layouts
  int rot;                      // 0: the RHT; 1: the Haar matrix
  bool compact;                 // staging slots sized from bps (hq_plan_set_compact_workspace)
  float* q;                     // Haar: Q (128 x 128 fp32, row-major, host), owned by the plan
  float* dq;                    // Haar: device copy (caller's memory): Q^T, then Q
};

namespace {

constexpr uint32_t kTagSign = 0x5349474Eu;  // "SIGN"

// Philox4x32-10 [Salmon et al., SC'11] on the host, for the sign vector of D.
void philox_host(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

int raw_bits(int lat) { return lat == HQ_E8 ? 16 : 0; }
uint64_t max_record_bits(int lat) { return (uint64_t)raw_bits(lat) + 128ull * 23ull; }

bool lattice_ok(int lat) { return lat >= HQ_Z && lat <= HQ_E8; }

hq_status dev_err(hipError_t e) { return e == hipSuccess ? HQ_OK : HQ_ERR_DEVICE; }

// A stream as the decode kernels read it: words in whole 16-byte groups from
// the 16-byte boundary below each chunk's first record, offsets as uint64.
bool stream_aligned(const uint32_t* words, const uint64_t* offsets) {
  return (((uintptr_t)words & 15u) == 0) && (((uintptr_t)offsets & 7u) == 0);
}

// The fp32 scale constants for alpha: the RHT folds 1/sqrt(128) in, the
// (orthonormal) Haar matrix does not.
void plan_scales(hq_plan_s* p, float alpha) {
  if (p->rot == 1) {
    p->c_enc = (float)(1.0 / (double)alpha);
    p->c_dec = alpha;
  } else {
    p->c_enc = (float)(1.0 / ((double)alpha * std::sqrt(128.0)));
    p->c_dec = (float)((double)alpha / std::sqrt(128.0));
  }
}

// The Haar rotation of a seed [reading of the QJL rotation the explainer
// compares with the RHT; Mezzadri, Notices AMS 54 (2007)]: G = 128 x 128
// standard normals, pair p from Philox4x32-10 (counter (p, 0, 0, "HAAR"),
// key = seed) by Box-Muller in double; Q = modified Gram-Schmidt of G's
// columns (dot products and updates in index order, double), so R has a
// positive diagonal and Q is Haar distributed; rounded to fp32, row-major.
constexpr uint32_t kTagHaar = 0x48414152u;  // "HAAR"
void haar_host(uint64_t seed, float* q32) {
  const int n = 128;
  double* g = new double[n * n];
  double* q = new double[n * n];
  for (uint32_t p = 0; p < (uint32_t)(n * n / 2); ++p) {
    uint32_t c[4] = {p, 0u, 0u, kTagHaar};
    philox_host(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const double u1 = ((double)c[0] + 1.0) / 4294967296.0;
    const double u2 = (double)c[1] / 4294967296.0;
    const double rad = std::sqrt(-2.0 * std::log(u1)), ang = 6.283185307179586 * u2;
    g[2 * p] = rad * std::cos(ang);
    g[2 * p + 1] = rad * std::sin(ang);
  }
  double v[128];
  for (int j = 0; j < n; ++j) {
    for (int i = 0; i < n; ++i) v[i] = g[i * n + j];
    for (int c = 0; c < j; ++c) {
      double r = 0.0;
      for (int i = 0; i < n; ++i) r = r + q[i * n + c] * v[i];
      for (int i = 0; i < n; ++i) v[i] = v[i] - r * q[i * n + c];
    }
    double nrm = 0.0;
    for (int i = 0; i < n; ++i) nrm = nrm + v[i] * v[i];
    nrm = std::sqrt(nrm);
    for (int i = 0; i < n; ++i) q[i * n + j] = v[i] / nrm;
  }
  for (int i = 0; i < n * n; ++i) q32[i] = (float)q[i];
  delete[] g;
  delete[] q;
}

// Workspace: the rotated tiles (fp32) of a Haar plan follow the codec regions.
// Staging slot words of the plan's encodes: full-size, or with a compact
// workspace sized from the plan's rate (hq_ws.h, slot_words_for).
uint32_t plan_slot_words(const hq_plan_s* p) {
  return p->compact ? hq::slot_words_for(p->bps) : (uint32_t)hq::kSlotWords;
}

// Haar plans: the rotated tiles (or queries) follow the codec's regions.
uint64_t rot_buffer_offset(const hq_plan_s* p, uint64_t n_tiles) {
  return hq::ws_align(hq::ws_bytes(n_tiles, plan_slot_words(p)));
}

// The signs of D (bit c of the 128: coordinate c is -1) in the two layouts the
// kernels read.  The lane holding vector v (coordinates 8v..8v+7) takes word
// v >> 2, in slot j = v & 3: for bf16 pairs, bit 15 - 4j - i is coordinate
// 8v + 2i and bit 31 - 4j - i coordinate 8v + 2i + 1 (i < 4); for fp32, bit
// 31 - 8j - i is coordinate 8v + i (i < 8).  A shift by 4j (8j) and a mask
// then give the lane its signs at the bit positions its arithmetic uses.
void sign_layouts(const uint32_t sgn[4], uint32_t sl16[4], uint32_t sl32[4]) {
  for (int q = 0; q < 4; ++q) sl16[q] = sl32[q] = 0;
  for (int c = 0; c < 128; ++c) {
    if (!((sgn[c >> 5] >> (c & 31)) & 1u)) continue;
    const int v = c >> 3, j = v & 3, i = c & 7;
    sl32[v >> 2] |= 1u << (31 - 8 * j - i);
    sl16[v >> 2] |= 1u << (((i & 1) ? 31 : 15) - 4 * j - (i >> 1));
  }
}

void fill_common(const hq_plan_s* p, uint32_t sl16[4], uint32_t sl32[4], uint32_t& k0, uint32_t& k1) {
  for (int q = 0; q < 4; ++q) {
    sl16[q] = p->sl16[q];
    sl32[q] = p->sl32[q];
  }
  k0 = (uint32_t)p->seed;
  k1 = (uint32_t)(p->seed >> 32);
}

// status: where the kernels record data errors (the workspace's own header
// unless given).
hq_status encode_impl(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles, bool dither,
                      uint64_t tile_base, uint32_t* words, uint64_t cap_words, uint64_t* offsets, uint8_t* k,
                      void* ws, void* stream, bool len_only, bool append = false, bool rotated = false,
                      hq::WsHeader* status = nullptr, bool noalloc_slots = false) {
  if (!plan) return HQ_ERR_ARG;
  if (!plan->has_alpha) return HQ_ERR_NOALPHA;
  if (dtype != HQ_F32 && dtype != HQ_BF16) return HQ_ERR_ARG;
  if (!ws) return HQ_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (!len_only && !offsets) return HQ_ERR_ARG;
  if (n_tiles == 0) {
    if (len_only || append) return HQ_OK;
    return dev_err(hq::launch_set_u64(offsets, 0, st));
  }
  if (!x) return HQ_ERR_ARG;
  if (!len_only && (!words || !k)) return HQ_ERR_ARG;
  if (((uintptr_t)x & 15u) != 0) return HQ_ERR_ARG;
  if (((uintptr_t)ws & 15u) != 0) return HQ_ERR_ARG;
  if (!len_only && ((((uintptr_t)words & 15u) != 0) || (((uintptr_t)offsets & 7u) != 0))) return HQ_ERR_ARG;
  // chunk indices are 32-bit (grid x)
  if (hq::ws_chunks(n_tiles) > 0x7FFFFFFFull) return HQ_ERR_ARG;
  hq::EncArgs a{};
  a.x = x;
  a.n_tiles = n_tiles;
  a.words = words;
  a.cap_words = cap_words;
  a.offsets = offsets;
  a.kout = k;
  fill_common(plan, a.sl16, a.sl32, a.key0, a.key1);
  a.c_enc = plan->c_enc;
  a.tile_base = tile_base;
  a.ws = status ? status : (hq::WsHeader*)ws;
  const uint32_t slot = noalloc_slots ? (uint32_t)hq::kSlotWords : plan_slot_words(plan);
  const hq::WsLayout lay = hq::ws_layout(n_tiles, slot);
  a.n_chunks = (uint32_t)hq::ws_chunks(n_tiles);
  a.agg = (uint32_t*)((char*)ws + lay.agg);
  a.E = (uint64_t*)((char*)ws + lay.E);
  a.loc = (uint32_t*)((char*)ws + lay.loc);
  a.tailw = (uint32_t*)((char*)ws + lay.tailw);
  a.stage = (uint32_t*)((char*)ws + lay.stage);
  a.slot_words = slot;
  a.partials = (unsigned long long*)a.E;
  a.base = append ? offsets : nullptr;
  int in = dtype == HQ_BF16 ? 1 : 0;
  if (plan->rot == 1) {  // the dense rotation first (skipped when the caller has it in the workspace)
    float* rbuf = (float*)((char*)ws + rot_buffer_offset(plan, n_tiles));
    if (!rotated) {
      hq::RotArgs r{};
      r.x = x;
      r.in_bf16 = dtype == HQ_BF16;
      r.y = rbuf;
      r.out_bf16 = 0;
      r.mt = plan->dq;  // Q^T: Mt[j][i] = Q[i][j]
      r.scale = 1.0f;
      r.n_tiles = n_tiles;
      if (hq::launch_rot(r, st) != hipSuccess) return HQ_ERR_DEVICE;
    }
    a.x = rbuf;
    a.x0 = x;
    a.x0_bf16 = dtype == HQ_BF16;
    in = 2;
  }
  return dev_err(hq::launch_encode(plan->lattice, dither, in, len_only, a, st));
}

hq_status decode_impl(hq_plan_t plan, const uint32_t* words, uint64_t n_words, const uint64_t* offsets,
                      const uint8_t* k, uint64_t n_tiles, bool dither, uint64_t tile_base, void* y,
                      hq_dtype out_dtype, void* ws, void* stream) {
  if (!plan) return HQ_ERR_ARG;
  if (!plan->has_alpha) return HQ_ERR_NOALPHA;
  if (out_dtype != HQ_F32 && out_dtype != HQ_BF16) return HQ_ERR_ARG;
  if (n_tiles == 0) return HQ_OK;
  if (!words || !offsets || !k || !y || !ws) return HQ_ERR_ARG;
  if (((uintptr_t)y & 15u) != 0 || ((uintptr_t)ws & 15u) != 0 || !stream_aligned(words, offsets)) return HQ_ERR_ARG;
  if (hq::ws_chunks(n_tiles) > 0x7FFFFFFFull) return HQ_ERR_ARG;
  hq::DecArgs a{};
  a.words = words;
  a.n_words = n_words;
  a.offsets = offsets;
  a.kin = k;
  a.n_tiles = n_tiles;
  a.y = y;
  fill_common(plan, a.sl16, a.sl32, a.key0, a.key1);
  a.c_dec = plan->c_dec;
  a.tile_base = tile_base;
  a.ws = (hq::WsHeader*)ws;
  const dim3 grid((uint32_t)hq::ws_chunks(n_tiles));
  if (plan->rot == 1) {  // the codes in the rotated domain, then the dense inverse rotation
    if (((uintptr_t)ws & 15u) != 0) return HQ_ERR_ARG;
    float* rbuf = (float*)((char*)ws + rot_buffer_offset(plan, n_tiles));
    a.y = rbuf;
    if (hq::launch_decode(plan->lattice, dither, hq::kOutRot, a, grid, (hipStream_t)stream) != hipSuccess)
      return HQ_ERR_DEVICE;
    hq::RotArgs r{};
    r.x = rbuf;
    r.in_bf16 = 0;
    r.y = y;
    r.out_bf16 = out_dtype == HQ_BF16;
    r.mt = plan->dq + 128 * 128;  // Q: Mt[j][i] = Q[j][i] gives Q^T u
    r.scale = plan->c_dec;
    r.n_tiles = n_tiles;
    return dev_err(hq::launch_rot(r, (hipStream_t)stream));
  }
  return dev_err(hq::launch_decode(plan->lattice, dither, out_dtype == HQ_BF16 ? hq::kOutBf16 : hq::kOutF32, a,
                                   grid, (hipStream_t)stream));
}

// Payload rate of x at alpha a on the device (bits per scalar); +inf when the
// step is too fine for the 2^20 code range.
hq_status rate_at(hq_plan_s* p, float a, const void* x, hq_dtype dtype, uint64_t n_tiles, bool dither,
                  uint64_t tile_base, void* ws, hipStream_t st, double* rate) {
  hq_plan_s q = *p;  // (shares the plan's rotation buffers; nothing is freed)
  q.has_alpha = true;
  q.alpha = a;
  plan_scales(&q, a);
  hq::WsHeader* h = (hq::WsHeader*)ws;
  // a Haar plan's rotated tiles are in the workspace already (hq_calibrate)
  hq_status s = encode_impl(&q, x, dtype, n_tiles, dither, tile_base, nullptr, 0, nullptr, nullptr, ws, st, true,
                            false, q.rot == 1);
  if (s != HQ_OK) return s;
  unsigned long long bits = 0;
  if (hipMemcpyAsync(&bits, &h->bits, sizeof(bits), hipMemcpyDeviceToHost, st) != hipSuccess) return HQ_ERR_DEVICE;
  s = hq_status_sync(ws, st);
  if (s == HQ_ERR_RANGE) {
    *rate = INFINITY;
    return HQ_ERR_RANGE;
  }
  if (s != HQ_OK) return s;
  *rate = (double)bits / ((double)n_tiles * 128.0);
  return HQ_OK;
}

// Container header fields, little-endian whatever the host.
constexpr uint32_t kHeaderMagic = 0x31535148u;  // "HQS1"
constexpr uint32_t kHeaderVersion = 1;

void put_le(uint8_t* p, int n, uint64_t v) {
  for (int i = 0; i < n; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

uint64_t get_le(const uint8_t* p, int n) {
  uint64_t v = 0;
  for (int i = 0; i < n; ++i) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

// CRC-32 of IEEE 802.3 (reflected polynomial 0xEDB88320, initial value and
// final xor 0xFFFFFFFF), one 256-entry table built on first use.
struct CrcTable {
  uint32_t t[256];
  CrcTable() {
    for (uint32_t i = 0; i < 256; ++i) {
      uint32_t c = i;
      for (int b = 0; b < 8; ++b) c = (c & 1u) ? 0xEDB88320u ^ (c >> 1) : c >> 1;
      t[i] = c;
    }
  }
};

uint32_t crc32_ieee(const uint8_t* p, size_t n) {
  static const CrcTable tab;  // initialised once, thread-safely
  const uint32_t* table = tab.t;
  uint32_t c = 0xFFFFFFFFu;
  for (size_t i = 0; i < n; ++i) c = table[(c ^ p[i]) & 0xFFu] ^ (c >> 8);
  return c ^ 0xFFFFFFFFu;
}

}  // namespace

// ---------------------------------------------------------------------------
// Workspace of hq_encode_noalloc: a fixed device array, one copy per GPU that
// runs it, held until the process ends.  Sized for HQ_NOALLOC_MAX_TILES tiles
// (the codec workspace layout of hq_ws.h; its header region is unused, the
// call records data errors in the caller's status block instead).  In host
// code `scratch` names a host-side stand-in: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[hq::ws_bytes(HQ_NOALLOC_MAX_TILES)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // per device: the device address of scratch, null until set up

// The current device's scratch address, looked up on the device's first call.
hq_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HQ_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HQ_ERR_DEVICE;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return HQ_OK;
}

}  // namespace

extern "C" {

hq_status hq_plan(hq_lattice lattice, int tile, float bps, uint64_t seed, hq_plan_t* out) {
  if (!out) return HQ_ERR_ARG;
  *out = nullptr;
  if (!lattice_ok(lattice) || tile != 128 || !(bps > 0.0f) || !std::isfinite(bps)) return HQ_ERR_ARG;
  hq_plan_s* p = new (std::nothrow) hq_plan_s{};
  if (!p) return HQ_ERR_ARG;
  p->lattice = lattice;
  p->bps = bps;
  p->seed = seed;
  uint32_t c[4] = {0u, 0u, 0u, kTagSign};
  philox_host(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  for (int i = 0; i < 4; ++i) p->sgn[i] = c[i];
  sign_layouts(p->sgn, p->sl16, p->sl32);
  *out = p;
  return HQ_OK;
}

hq_status hq_plan_set_alpha(hq_plan_t plan, float alpha) {
  if (!plan || !(alpha > 0.0f) || !std::isfinite(alpha)) return HQ_ERR_ARG;
  plan->alpha = alpha;
  plan_scales(plan, alpha);
  plan->has_alpha = true;
  return HQ_OK;
}

hq_status hq_plan_get(hq_plan_t plan, float* alpha, float* c_enc, float* c_dec) {
  if (!plan) return HQ_ERR_ARG;
  if (!plan->has_alpha) return HQ_ERR_NOALPHA;
  if (alpha) *alpha = plan->alpha;
  if (c_enc) *c_enc = plan->c_enc;
  if (c_dec) *c_dec = plan->c_dec;
  return HQ_OK;
}

void hq_plan_destroy(hq_plan_t plan) {
  if (plan) delete[] plan->q;
  delete plan;
}

size_t hq_workspace_bytes(hq_plan_t plan, uint64_t n_tiles) {
  if (plan && plan->rot == 1) return (size_t)(rot_buffer_offset(plan, n_tiles) + 512ull * n_tiles);
  return (size_t)hq::ws_bytes(n_tiles, plan ? plan_slot_words(plan) : (uint32_t)hq::kSlotWords);
}

hq_status hq_plan_set_compact_workspace(hq_plan_t plan, int on) {
  if (!plan || (on != 0 && on != 1)) return HQ_ERR_ARG;
  plan->compact = on == 1;
  return HQ_OK;
}

size_t hq_rotation_bytes(void) { return 2 * 128 * 128 * sizeof(float); }

hq_status hq_plan_set_rotation(hq_plan_t plan, int kind, void* dev_buf, void* stream) {
  if (!plan || (kind != 0 && kind != 1)) return HQ_ERR_ARG;
  if (kind == 0) {
    plan->rot = 0;
    plan->dq = nullptr;
  } else {
    if (!dev_buf || ((uintptr_t)dev_buf & 15u) != 0) return HQ_ERR_ARG;
    if (!plan->q) {
      plan->q = new (std::nothrow) float[128 * 128];
      if (!plan->q) return HQ_ERR_ARG;
      haar_host(plan->seed, plan->q);
    }
    float* both = new (std::nothrow) float[2 * 128 * 128];
    if (!both) return HQ_ERR_ARG;
    for (int i = 0; i < 128; ++i)
      for (int j = 0; j < 128; ++j) {
        both[j * 128 + i] = plan->q[i * 128 + j];    // Q^T (the forward rotation's Mt)
        both[16384 + i * 128 + j] = plan->q[i * 128 + j];  // Q (the inverse's Mt)
      }
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e1 = hipMemcpyAsync(dev_buf, both, hq_rotation_bytes(), hipMemcpyHostToDevice, st);
    const hipError_t e2 = hipStreamSynchronize(st);
    delete[] both;
    if (e1 != hipSuccess || e2 != hipSuccess) return HQ_ERR_DEVICE;
    plan->rot = 1;
    plan->dq = (float*)dev_buf;
  }
  if (plan->has_alpha) plan_scales(plan, plan->alpha);
  return HQ_OK;
}

hq_status hq_plan_get_rotation(hq_plan_t plan, int* kind, float* q) {
  if (!plan) return HQ_ERR_ARG;
  if (kind) *kind = plan->rot;
  if (q) {
    if (plan->q) {
      for (int i = 0; i < 128 * 128; ++i) q[i] = plan->q[i];
    } else {
      haar_host(plan->seed, q);  // (host only: the matrix the seed would give)
    }
  }
  return HQ_OK;
}

uint64_t hq_encode_bound_words(hq_plan_t plan, uint64_t n_tiles) {
  const int lat = plan ? plan->lattice : HQ_E8;
  return (n_tiles * max_record_bits(lat) + 31) / 32;
}

hq_status hq_encode(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles, uint32_t* words,
                    uint64_t cap_words, uint64_t* offsets, uint8_t* k, void* ws, void* stream) {
  return encode_impl(plan, x, dtype, n_tiles, false, 0, words, cap_words, offsets, k, ws, stream, false);
}

hq_status hq_encode_noalloc(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles, uint32_t* words,
                            uint64_t cap_words, uint64_t* offsets, uint8_t* k, void* status, void* stream) {
  if (!plan) return HQ_ERR_ARG;
  if (!plan->has_alpha) return HQ_ERR_NOALPHA;
  if (plan->rot != 0) return HQ_ERR_ARG;  // the scratch holds no rotated tiles
  if (n_tiles > HQ_NOALLOC_MAX_TILES) return HQ_ERR_ARG;
  if (!status || ((uintptr_t)status & 15u) != 0) return HQ_ERR_ARG;
  void* ws = nullptr;
  const hq_status s = scratch_address(&ws);
  if (s != HQ_OK) return s;
  return encode_impl(plan, x, dtype, n_tiles, false, 0, words, cap_words, offsets, k, ws, stream, false, false, false,
                     (hq::WsHeader*)status, true);
}

hq_status hq_kv_encode(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles, uint64_t tile_base,
                       uint32_t* words, uint64_t cap_words, uint64_t* offsets, uint8_t* k, void* ws, void* stream) {
  return encode_impl(plan, x, dtype, n_tiles, true, tile_base, words, cap_words, offsets, k, ws, stream, false);
}

hq_status hq_append(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles, uint32_t* words,
                    uint64_t cap_words, uint64_t* offsets, uint8_t* k, uint64_t n_prev, void* ws, void* stream) {
  if (!offsets || !k) return HQ_ERR_ARG;
  return encode_impl(plan, x, dtype, n_tiles, false, 0, words, cap_words, offsets + n_prev, k + n_prev, ws, stream,
                     false, n_prev > 0);
}

hq_status hq_kv_append(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles, uint64_t tile_base,
                       uint32_t* words, uint64_t cap_words, uint64_t* offsets, uint8_t* k, uint64_t n_prev, void* ws,
                       void* stream) {
  if (!offsets || !k) return HQ_ERR_ARG;
  return encode_impl(plan, x, dtype, n_tiles, true, tile_base, words, cap_words, offsets + n_prev, k + n_prev, ws,
                     stream, false, n_prev > 0);
}

hq_status hq_decode(hq_plan_t plan, const uint32_t* words, uint64_t n_words, const uint64_t* offsets,
                    const uint8_t* k, uint64_t n_tiles, void* y, hq_dtype out_dtype, void* ws, void* stream) {
  return decode_impl(plan, words, n_words, offsets, k, n_tiles, false, 0, y, out_dtype, ws, stream);
}

hq_status hq_kv_decode(hq_plan_t plan, const uint32_t* words, uint64_t n_words, const uint64_t* offsets,
                       const uint8_t* k, uint64_t n_tiles, uint64_t tile_base, void* y, hq_dtype out_dtype,
                       void* ws, void* stream) {
  return decode_impl(plan, words, n_words, offsets, k, n_tiles, true, tile_base, y, out_dtype, ws, stream);
}

size_t hq_kv_scores_workspace_bytes(hq_plan_t plan, uint32_t n_heads, uint64_t tiles_per_head, uint32_t qph) {
  const uint64_t n = (uint64_t)n_heads * tiles_per_head;
  if (plan && plan->rot == 1) {  // the rotated queries follow the codec's regions
    const uint64_t a = hq_workspace_bytes(plan, n), b = rot_buffer_offset(plan, n) + 512ull * n_heads * qph;
    return (size_t)(a > b ? a : b);
  }
  return hq_workspace_bytes(plan, n);
}

hq_status hq_kv_scores(hq_plan_t plan, const uint32_t* words, uint64_t n_words, const uint64_t* offsets,
                       const uint8_t* k, uint32_t n_heads, uint64_t tiles_per_head, uint64_t tile_base,
                       const float* q, uint32_t qph, float* scores, void* ws, void* stream) {
  if (!plan) return HQ_ERR_ARG;
  if (!plan->has_alpha) return HQ_ERR_NOALPHA;
  if (plan->rot != 0 && plan->rot != 1) return HQ_ERR_ARG;
  if (qph == 0 || qph > 16) return HQ_ERR_ARG;
  if (n_heads == 0 || tiles_per_head == 0) return HQ_OK;
  if (!words || !offsets || !k || !q || !scores || !ws) return HQ_ERR_ARG;
  const uint64_t cph = (tiles_per_head + hq::kChunkTiles - 1) / hq::kChunkTiles;
  if (cph > 0x7FFFFFFFull || n_heads > 65535u) return HQ_ERR_ARG;
  if (!stream_aligned(words, offsets) || ((uintptr_t)ws & 15u) != 0) return HQ_ERR_ARG;
  if (plan->rot == 1 && ((((uintptr_t)q | (uintptr_t)ws) & 15u) != 0)) return HQ_ERR_ARG;
  hq::DecArgs a{};
  a.words = words;
  a.n_words = n_words;
  a.offsets = offsets;
  a.kin = k;
  a.n_tiles = (uint64_t)n_heads * tiles_per_head;
  fill_common(plan, a.sl16, a.sl32, a.key0, a.key1);
  a.c_dec = plan->c_dec;
  a.tile_base = tile_base;
  a.ws = (hq::WsHeader*)ws;
  a.q = q;
  a.scores = scores;
  a.qph = qph;
  a.tiles_per_head = tiles_per_head;
  if (plan->rot == 1) {  // q~ = Q q (fp32 chains, as the encoder rotates the keys) into the workspace
    float* qr = (float*)((char*)ws + rot_buffer_offset(plan, a.n_tiles));
    hq::RotArgs r{};
    r.x = q;
    r.in_bf16 = 0;
    r.y = qr;
    r.out_bf16 = 0;
    r.mt = plan->dq;  // Q^T: Mt[j][i] = Q[i][j]
    r.scale = 1.0f;
    r.n_tiles = (uint64_t)n_heads * qph;
    if (hq::launch_rot(r, (hipStream_t)stream) != hipSuccess) return HQ_ERR_DEVICE;
    a.q = qr;
    a.q_rot = 1;
  }
  return dev_err(hq::launch_decode(plan->lattice, true, hq::kOutScores, a, dim3((uint32_t)cph, n_heads),
                                   (hipStream_t)stream));
}

size_t hq_gemv_workspace_bytes(uint64_t rows, uint64_t cols, uint32_t nb) {
  const uint64_t xr = hq::ws_align(4ull * nb * cols);
  return (size_t)(sizeof(hq::WsHeader) + xr + 4ull * nb * rows * (cols / 128));
}

hq_status hq_gemv(hq_plan_t plan, const uint32_t* words, uint64_t n_words, const uint64_t* offsets,
                  const uint8_t* k, uint64_t rows, uint64_t cols, const float* x, uint32_t nb, float* y,
                  void* ws, void* stream) {
  if (!plan) return HQ_ERR_ARG;
  if (!plan->has_alpha) return HQ_ERR_NOALPHA;
  if (plan->rot != 0) return HQ_ERR_ARG;  // fused paths use the RHT
  if (cols == 0 || cols % 128 || nb == 0 || nb > 16) return HQ_ERR_ARG;
  if (rows == 0) return HQ_OK;
  if (!words || !offsets || !k || !x || !y || !ws) return HQ_ERR_ARG;
  if (((uintptr_t)x & 15u) != 0 || ((uintptr_t)ws & 15u) != 0 || !stream_aligned(words, offsets)) return HQ_ERR_ARG;
  const uint64_t nblk = cols / 128, n_tiles = rows * nblk;
  if (rows > 0xFFFFFFFFull || n_tiles / nblk != rows || n_tiles > 0xFFFFFFFFull || (uint64_t)nb * rows > 0xFFFFFFFFull ||
      (uint64_t)nb * nblk > 0xFFFFFFFFull)
    return HQ_ERR_ARG;
  float* xr = (float*)((char*)ws + sizeof(hq::WsHeader));
  float* dots = (float*)((char*)xr + hq::ws_align(4ull * nb * cols));
  hq::DecArgs d{};
  d.words = words;
  d.n_words = n_words;
  d.offsets = offsets;
  d.kin = k;
  d.n_tiles = n_tiles;
  fill_common(plan, d.sl16, d.sl32, d.key0, d.key1);
  d.c_dec = plan->c_dec;
  d.ws = (hq::WsHeader*)ws;
  d.xr = xr;
  d.dots = dots;
  d.nb = nb;
  d.nblk = (uint32_t)nblk;
  hq::GemvArgs g{};
  g.x = x;
  g.xr = xr;
  g.dots = dots;
  g.y = y;
  g.rows = (uint32_t)rows;
  g.nblk = (uint32_t)nblk;
  g.nb = nb;
  for (int i = 0; i < 4; ++i) g.sl32[i] = d.sl32[i];
  g.c_dec = plan->c_dec;
  return dev_err(hq::launch_gemv(plan->lattice, d, g, (hipStream_t)stream));
}

namespace {
struct GemmShape {
  uint32_t nbp, splits, per;
  uint64_t xp_bytes, part_bytes;
};
GemmShape gemm_shape(uint64_t rows, uint64_t cols, uint32_t nb) {
  GemmShape g{};
  const uint64_t nblk = cols / 128, ntn = (rows + 31) / 32;
  g.nbp = nb <= 32 ? 32u : 64u;
  uint64_t want = ntn >= 2048 ? 1 : (2048 + ntn - 1) / ntn;  // about 2048 work-groups
  if (want > nblk) want = nblk;
  if (want < 1) want = 1;
  g.per = (uint32_t)((nblk + want - 1) / want);
  g.splits = g.per ? (uint32_t)((nblk + g.per - 1) / g.per) : 1u;
  g.xp_bytes = hq::ws_align(2ull * 2ull * g.nbp * cols);
  g.part_bytes = g.splits > 1 ? 4ull * g.splits * g.nbp * rows : 0ull;
  return g;
}
}  // namespace

size_t hq_gemm_workspace_bytes(uint64_t rows, uint64_t cols, uint32_t nb) {
  const GemmShape g = gemm_shape(rows, cols, nb);
  return (size_t)(sizeof(hq::WsHeader) + g.xp_bytes + g.part_bytes);
}

hq_status hq_gemm(hq_plan_t plan, const uint32_t* words, uint64_t n_words, const uint64_t* offsets, const uint8_t* k,
                  uint64_t rows, uint64_t cols, const float* x, uint32_t nb, float* y, void* ws, void* stream) {
  if (!plan) return HQ_ERR_ARG;
  if (!plan->has_alpha) return HQ_ERR_NOALPHA;
  if (plan->rot != 0) return HQ_ERR_ARG;  // fused paths use the RHT
  if (plan->lattice == HQ_A2) return HQ_ERR_ARG;  // its codes are not integers
  if (cols == 0 || cols % 128 || nb == 0 || nb > hq::kGemmMaxVec) return HQ_ERR_ARG;
  if (rows == 0) return HQ_OK;
  if (!words || !offsets || !k || !x || !y || !ws) return HQ_ERR_ARG;
  if (((uintptr_t)x & 15u) != 0 || ((uintptr_t)ws & 15u) != 0 || !stream_aligned(words, offsets)) return HQ_ERR_ARG;
  const uint64_t nblk = cols / 128;
  if (rows > 0x7FFFFFFFull || nblk > 0xFFFFFFFFull || rows * nblk / nblk != rows || (uint64_t)nb * rows > 0xFFFFFFFFull)
    return HQ_ERR_ARG;
  const GemmShape sh = gemm_shape(rows, cols, nb);
  if (sh.splits > 65535u) return HQ_ERR_ARG;
  hq::GemmArgs g{};
  g.words = words;
  g.n_words = n_words;
  g.offsets = offsets;
  g.k = k;
  g.ws = (hq::WsHeader*)ws;
  g.x = x;
  g.xp = (uint16_t*)((char*)ws + sizeof(hq::WsHeader));
  g.part = (float*)((char*)ws + sizeof(hq::WsHeader) + sh.xp_bytes);
  g.y = y;
  g.rows = (uint32_t)rows;
  g.nblk = (uint32_t)nblk;
  g.nb = nb;
  g.nbp = sh.nbp;
  g.splits = sh.splits;
  g.per = sh.per;
  uint32_t sl16[4], k0, k1;
  fill_common(plan, sl16, g.sl32, k0, k1);
  g.c_dec = plan->c_dec;
  return dev_err(hq::launch_gemm(plan->lattice, g, (hipStream_t)stream));
}

namespace {
// The attention workspace: [header][partials][per query 128 floats: the
// rotated queries, then the pre-image of the output (dense rotation only)].
uint64_t attn_qbuf_offset(uint32_t n_heads, uint64_t seq, uint32_t qph) {
  const uint64_t groups = (seq + hq::kAttnChunks * hq::kChunkTiles - 1) / (hq::kAttnChunks * hq::kChunkTiles);
  return hq::ws_align(sizeof(hq::WsHeader) + 4ull * n_heads * groups * qph * hq::kAttnPart);
}
}  // namespace

size_t hq_kv_attention_workspace_bytes(uint32_t n_heads, uint64_t seq, uint32_t qph) {
  return (size_t)(attn_qbuf_offset(n_heads, seq, qph) + 512ull * n_heads * qph);
}

hq_status hq_kv_attention(hq_plan_t plan_k, const uint32_t* k_words, uint64_t k_n_words, const uint64_t* k_offsets,
                          const uint8_t* k_k, uint64_t k_tile_base, hq_plan_t plan_v, const uint32_t* v_words,
                          uint64_t v_n_words, const uint64_t* v_offsets, const uint8_t* v_k, uint64_t v_tile_base,
                          uint32_t n_heads, uint64_t seq, const float* q, uint32_t qph, float scale, float* out,
                          void* ws, void* stream) {
  if (!plan_k || !plan_v) return HQ_ERR_ARG;
  if (!plan_k->has_alpha || !plan_v->has_alpha) return HQ_ERR_NOALPHA;
  if (plan_k->rot != plan_v->rot || (plan_k->rot != 0 && plan_k->rot != 1)) return HQ_ERR_ARG;
  if (plan_k->lattice != plan_v->lattice || plan_k->seed != plan_v->seed) return HQ_ERR_ARG;
  if (qph == 0 || qph > 16 || !(scale == scale) || scale - scale != 0.0f) return HQ_ERR_ARG;
  if (n_heads == 0) return HQ_OK;
  if (seq == 0 || !k_words || !k_offsets || !k_k || !v_words || !v_offsets || !v_k || !q || !out || !ws)
    return HQ_ERR_ARG;
  if (((uintptr_t)ws & 15u) != 0) return HQ_ERR_ARG;
  if (!stream_aligned(k_words, k_offsets) || !stream_aligned(v_words, v_offsets)) return HQ_ERR_ARG;
  if (plan_k->rot == 1 && ((((uintptr_t)q | (uintptr_t)out) & 15u) != 0)) return HQ_ERR_ARG;
  const uint64_t groups = (seq + hq::kAttnChunks * hq::kChunkTiles - 1) / (hq::kAttnChunks * hq::kChunkTiles);
  if (n_heads > 65535u || groups > 0x7FFFFFFFull || seq > (1ull << 40)) return HQ_ERR_ARG;
  hq::AttnArgs a{};
  a.kw = k_words;
  a.kn = k_n_words;
  a.ko = k_offsets;
  a.kk = k_k;
  a.ktb = k_tile_base;
  a.ck = plan_k->c_dec;
  a.vw = v_words;
  a.vn = v_n_words;
  a.vo = v_offsets;
  a.vk = v_k;
  a.vtb = v_tile_base;
  a.cv = plan_v->c_dec;
  uint32_t sl16[4];
  fill_common(plan_k, sl16, a.sl32, a.key0, a.key1);
  a.q = q;
  a.qph = qph;
  a.scale = scale;
  a.seq = seq;
  a.n_groups = (uint32_t)groups;
  a.ws = (hq::WsHeader*)ws;
  a.part = (float*)((char*)ws + sizeof(hq::WsHeader));
  a.out = out;
  if (plan_k->rot == 0) return dev_err(hq::launch_attention(plan_k->lattice, a, n_heads, (hipStream_t)stream));
  // dense rotation: q~ = Q q into the workspace; the combine leaves c_dec_V A / L
  // there (the rotated queries are consumed by then) and rot_k applies Q^T
  const hipStream_t st = (hipStream_t)stream;
  float* qb = (float*)((char*)ws + attn_qbuf_offset(n_heads, seq, qph));
  hq::RotArgs r{};
  r.x = q;
  r.y = qb;
  r.mt = plan_k->dq;  // Q^T: Mt[j][i] = Q[i][j]
  r.scale = 1.0f;
  r.n_tiles = (uint64_t)n_heads * qph;
  if (hq::launch_rot(r, st) != hipSuccess) return HQ_ERR_DEVICE;
  a.q = qb;
  a.q_rot = 1;
  a.rot_out = qb;
  if (hq::launch_attention(plan_k->lattice, a, n_heads, st) != hipSuccess) return HQ_ERR_DEVICE;
  r.x = qb;
  r.y = out;
  r.mt = plan_v->dq + 128 * 128;  // Q: Mt[j][i] = Q[j][i] gives Q^T y
  return dev_err(hq::launch_rot(r, st));
}

size_t hq_side_bytes(uint64_t n_tiles) { return (size_t)(96ull * ((n_tiles + 31) / 32)); }

hq_status hq_side_pack(const uint64_t* offsets, const uint8_t* k, uint64_t n_tiles, void* side, void* ws,
                       void* stream) {
  if (n_tiles == 0) return HQ_OK;
  if (!offsets || !k || !side || !ws) return HQ_ERR_ARG;
  if (((uintptr_t)side & 15u) != 0 || ((uintptr_t)offsets & 7u) != 0) return HQ_ERR_ARG;
  if ((n_tiles + 255) / 256 > 0x7FFFFFFFull) return HQ_ERR_ARG;
  return dev_err(hq::launch_side(true, offsets, k, nullptr, n_tiles, (uint8_t*)side, nullptr, nullptr,
                                 (hq::WsHeader*)ws, (hipStream_t)stream));
}

hq_status hq_side_unpack(const void* side, uint64_t n_tiles, uint64_t* offsets, uint8_t* k, void* stream) {
  if (!offsets) return HQ_ERR_ARG;
  if (n_tiles == 0) return dev_err(hq::launch_set_u64(offsets, 0, (hipStream_t)stream));
  if (!side || !k) return HQ_ERR_ARG;
  if (((uintptr_t)side & 15u) != 0 || ((uintptr_t)offsets & 7u) != 0) return HQ_ERR_ARG;
  if ((n_tiles + 255) / 256 > 0x7FFFFFFFull) return HQ_ERR_ARG;
  return dev_err(hq::launch_side(false, nullptr, nullptr, (const uint8_t*)side, n_tiles, nullptr, offsets, k, nullptr,
                                 (hipStream_t)stream));
}

hq_status hq_header_write(hq_plan_t plan, int dithered, uint64_t tile_base, uint64_t n_tiles, uint64_t total_bits,
                          int compact_side, void* out) {
  if (!plan || !out) return HQ_ERR_ARG;
  if (!plan->has_alpha) return HQ_ERR_NOALPHA;
  uint8_t h[HQ_HEADER_BYTES] = {};
  put_le(h + 0, 4, kHeaderMagic);
  put_le(h + 4, 2, kHeaderVersion);
  h[6] = (uint8_t)plan->lattice;
  h[7] = (uint8_t)((dithered ? 1u : 0u) | (compact_side ? 2u : 0u) | (plan->rot == 1 ? 4u : 0u));
  put_le(h + 8, 4, 128u);
  uint32_t ab, bb;
  std::memcpy(&ab, &plan->alpha, 4);
  std::memcpy(&bb, &plan->bps, 4);
  put_le(h + 12, 4, ab);
  put_le(h + 16, 4, bb);
  put_le(h + 24, 8, plan->seed);
  put_le(h + 32, 8, tile_base);
  put_le(h + 40, 8, n_tiles);
  put_le(h + 48, 8, total_bits);
  put_le(h + 60, 4, crc32_ieee(h, 60));
  std::memcpy(out, h, HQ_HEADER_BYTES);
  return HQ_OK;
}

hq_status hq_header_read(const void* in, hq_header_info* info) {
  if (!in || !info) return HQ_ERR_ARG;
  const uint8_t* h = (const uint8_t*)in;
  if (get_le(h + 0, 4) != kHeaderMagic || get_le(h + 4, 2) != kHeaderVersion) return HQ_ERR_CORRUPT;
  if (get_le(h + 60, 4) != crc32_ieee(h, 60)) return HQ_ERR_CORRUPT;
  if (!lattice_ok(h[6]) || (h[7] & ~7u) != 0 || get_le(h + 8, 4) != 128u) return HQ_ERR_CORRUPT;
  const uint32_t ab = (uint32_t)get_le(h + 12, 4), bb = (uint32_t)get_le(h + 16, 4);
  std::memcpy(&info->alpha, &ab, 4);
  std::memcpy(&info->bps, &bb, 4);
  if (!(info->alpha > 0.0f) || !std::isfinite(info->alpha) || !(info->bps > 0.0f) || !std::isfinite(info->bps))
    return HQ_ERR_CORRUPT;
  info->lattice = (hq_lattice)h[6];
  info->dithered = h[7] & 1u;
  info->compact_side = (h[7] >> 1) & 1u;
  info->rotation = (h[7] >> 2) & 1u;
  info->tile = 128;
  info->seed = get_le(h + 24, 8);
  info->tile_base = get_le(h + 32, 8);
  info->n_tiles = get_le(h + 40, 8);
  info->total_bits = get_le(h + 48, 8);
  return HQ_OK;
}

hq_status hq_plan_from_header(const void* in, hq_plan_t* out) {
  if (!out) return HQ_ERR_ARG;
  *out = nullptr;
  hq_header_info info;
  hq_status s = hq_header_read(in, &info);
  if (s != HQ_OK) return s;
  s = hq_plan(info.lattice, info.tile, info.bps, info.seed, out);
  if (s != HQ_OK) return s;
  return hq_plan_set_alpha(*out, info.alpha);
}

hq_status hq_status_sync(void* ws, void* stream) {
  if (!ws) return HQ_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  hq::WsHeader* h = (hq::WsHeader*)ws;
  uint32_t bits = 0;
  if (hipMemcpyAsync(&bits, &h->status, sizeof(bits), hipMemcpyDeviceToHost, st) != hipSuccess) return HQ_ERR_DEVICE;
  if (hipStreamSynchronize(st) != hipSuccess) return HQ_ERR_DEVICE;
  if (bits == 0) return HQ_OK;
  if (hipMemsetAsync(&h->status, 0, sizeof(uint32_t), st) != hipSuccess) return HQ_ERR_DEVICE;
  if (hipStreamSynchronize(st) != hipSuccess) return HQ_ERR_DEVICE;
  for (int c = 1; c < 32; ++c)
    if (bits & (1u << c)) return (hq_status)c;
  return HQ_ERR_DEVICE;
}

const char* hq_status_str(hq_status s) {
  switch (s) {
    case HQ_OK: return "ok";
    case HQ_ERR_ARG: return "invalid argument";
    case HQ_ERR_NONFINITE: return "non-finite input";
    case HQ_ERR_RANGE: return "scaled coordinate out of range (alpha too small)";
    case HQ_ERR_CAPACITY: return "stream exceeds the word capacity";
    case HQ_ERR_CORRUPT: return "corrupt stream";
    case HQ_ERR_DEVICE: return "HIP runtime error";
    case HQ_ERR_NOALPHA: return "plan has no alpha";
  }
  return "unknown status";
}

// Bisection [reading of Methodology 3]: start from the high-resolution
// estimate alpha0 = sqrt(2 pi e) sigma / (nu 2^R) (sigma the RMS of x, nu the
// per-dimension cell edge of the embedding), bracket the target in log2 alpha
// from floor(log2 alpha0) -/+ 4 in steps of 4, then bisect on the exact payload
// rate until within 0.002 bps, at most 40 times.  Each trial alpha is
// fp32(2^mid); the closest rate wins, ties to the larger alpha.
hq_status hq_calibrate(hq_plan_t plan, const void* x, hq_dtype dtype, uint64_t n_tiles, int dithered,
                       uint64_t tile_base, void* ws, void* stream, float* alpha_out, double* bps_out) {
  if (!plan || !x || !ws || n_tiles == 0) return HQ_ERR_ARG;
  if (dtype != HQ_F32 && dtype != HQ_BF16) return HQ_ERR_ARG;
  if (((uintptr_t)x & 15u) != 0 || ((uintptr_t)ws & 15u) != 0) return HQ_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  hq::WsHeader* h = (hq::WsHeader*)ws;
  const uint64_t n = n_tiles * 128ull;
  uint32_t* partials = (uint32_t*)((char*)ws + sizeof(hq::WsHeader));
  const uint64_t chunks = hq::ws_chunks(n_tiles);
  if (hq::launch_absmax(x, dtype == HQ_BF16, n, partials, (uint32_t)(chunks < 1024 ? chunks : 1024), &h->absmax, st) !=
      hipSuccess)
    return HQ_ERR_DEVICE;
  uint32_t amax_bits = 0;
  if (hipMemcpyAsync(&amax_bits, &h->absmax, sizeof(uint32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return HQ_ERR_DEVICE;
  if (hipStreamSynchronize(st) != hipSuccess) return HQ_ERR_DEVICE;
  if (amax_bits >= 0x7F800000u) return HQ_ERR_NONFINITE;
  if (amax_bits == 0u) return HQ_ERR_ARG;
  float amax;
  std::memcpy(&amax, &amax_bits, sizeof(amax));
  if (plan->rot == 1) {  // the dense rotation once; every trial then scales it
    hq::RotArgs r{};
    r.x = x;
    r.in_bf16 = dtype == HQ_BF16;
    r.y = (float*)((char*)ws + rot_buffer_offset(plan, n_tiles));
    r.out_bf16 = 0;
    r.mt = plan->dq;
    r.scale = 1.0f;
    r.n_tiles = n_tiles;
    if (hq::launch_rot(r, st) != hipSuccess) return HQ_ERR_DEVICE;
  }
  // The bracket starts from exact integers only: the binary exponent eA of
  // max |x|, eN = ceil(log2 N) and floor(bps); the high-resolution estimate
  // sqrt(2 pi e) sigma / (nu 2^R), with sigma in [max/sqrt N, max] and nu in
  // [1, 2], lies within [eA - floor(R) - 4 - ceil(eN/2), eA - floor(R) + 4]
  // in log2, and the bracket widens by 4 octaves while it does not hold the
  // target.  Nothing here depends on the order of a floating-point sum, so
  // every exact evaluation of the rate takes the same path.
  int eA1 = 0;
  std::frexp((double)amax, &eA1);  // floor(log2 amax) = eA1 - 1
  int eN = 0;
  while ((1ull << eN) < n) ++eN;
  const double eA = (double)(eA1 - 1), Rf = std::floor((double)plan->bps);
  const double target = (double)plan->bps;
  double lo = eA - Rf - 4.0 - (double)((eN + 1) / 2), hi = eA - Rf + 4.0;
  float best_a = 0.0f;
  double best_r = 0.0, best_err = INFINITY;
  auto consider = [&](float a, double r) {
    const double e = std::fabs(r - target);
    if (e < best_err || (e == best_err && a > best_a)) {
      best_err = e;
      best_a = a;
      best_r = r;
    }
  };
  double r = 0.0;
  for (int g = 0; g < 16; ++g) {
    const float a = (float)std::exp2(lo);
    const hq_status s = rate_at(plan, a, x, dtype, n_tiles, dithered != 0, tile_base, ws, st, &r);
    if (s != HQ_OK && s != HQ_ERR_RANGE) return s;
    if (s == HQ_OK) consider(a, r);
    if (r >= target) break;
    lo -= 4.0;
  }
  for (int g = 0; g < 16; ++g) {
    const float a = (float)std::exp2(hi);
    const hq_status s = rate_at(plan, a, x, dtype, n_tiles, dithered != 0, tile_base, ws, st, &r);
    if (s != HQ_OK && s != HQ_ERR_RANGE) return s;
    if (s == HQ_OK) consider(a, r);
    if (r <= target) break;
    hi += 4.0;
  }
  for (int it = 0; it < 40 && best_err > 0.002; ++it) {
    const double mid = 0.5 * (lo + hi);
    const float a = (float)std::exp2(mid);
    const hq_status s = rate_at(plan, a, x, dtype, n_tiles, dithered != 0, tile_base, ws, st, &r);
    if (s != HQ_OK && s != HQ_ERR_RANGE) return s;
    if (s == HQ_OK) consider(a, r);
    if (r > target) lo = mid;
    else hi = mid;
  }
  if (!(best_a > 0.0f)) return HQ_ERR_RANGE;
  hq_plan_set_alpha(plan, best_a);
  if (alpha_out) *alpha_out = best_a;
  if (bps_out) *bps_out = best_r;
  return HQ_OK;
}

}  // extern "C"
