"""CPU oracle for the Muon optimizer step — TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the bench's CPU-baseline leg may import this
package. The HIP library never calls it, and it shares no code with the HIP
library: it is a plain, slow, float64 NumPy restatement of what the pages
describe, used to check the GPU path.
"""

from .muon_oracle import *  # noqa: F401,F403
