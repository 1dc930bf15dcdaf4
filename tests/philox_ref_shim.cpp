// Test-only shim: exposes the host-callable Philox4x32-10 of the ROCm rocRAND headers
// (an implementation independent of the oracle) to ctypes.
#include <rocrand/rocrand_philox4x32_10.h>
struct Exposed : rocrand_device::philox4x32_10_engine { using rocrand_device::philox4x32_10_engine::ten_rounds; };
extern "C" void ref_philox(const unsigned* c, const unsigned* k, unsigned* o) {
  Exposed e;
  uint4 ctr; ctr.x=c[0]; ctr.y=c[1]; ctr.z=c[2]; ctr.w=c[3];
  uint2 key; key.x=k[0]; key.y=k[1];
  uint4 r = e.ten_rounds(ctr, key);
  o[0]=r.x; o[1]=r.y; o[2]=r.z; o[3]=r.w;
}
