// Library-wide entry points of libdcp: error names and ABI version.
#include "dcp_common.h"

extern "C" const char* dcp_strerror(int code) {
  switch (code) {
    case DCP_OK: return "DCP_OK: success";
    case DCP_EINVAL: return "DCP_EINVAL: invalid argument";
    case DCP_EUNSUPPORTED: return "DCP_EUNSUPPORTED: shape not supported by the kernels";
    case DCP_EHIP: return "DCP_EHIP: HIP call or kernel launch failed";
    case DCP_ERANGE: return "DCP_ERANGE: device data out of range";
    case DCP_ESCRATCH: return "DCP_ESCRATCH: the shape needs more scratch than the fixed no-allocation buffer holds";
    default: return "unknown dcp status code";
  }
}

extern "C" int dcp_abi_version(void) { return 9; }
