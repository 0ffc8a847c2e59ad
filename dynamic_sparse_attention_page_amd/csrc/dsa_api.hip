// Library-wide entry points of libdsa: status names and version.
#include "dsa_host.hpp"

extern "C" const char* dsa_status_str(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "null pointer";
    case DSA_ERR_SHAPE: return "bad shape or size";
    case DSA_ERR_DTYPE: return "unknown dtype";
    case DSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case DSA_ERR_LAUNCH: return "kernel launch failed";
    case DSA_ERR_SCRATCH: return "needs more than the fixed no-allocation scratch";
  }
  return "unknown status";
}

extern "C" int dsa_version(void) { return 100; }
